// Host-side internals of the C ABI (not part of the public interface).
#pragma once

#include <cstdint>

namespace dbs {

// perm[new] = old for the Gilbert curve / cuboid order (host, shape only).
void gilbert3d(int T, int H, int W, int prefix, int32_t* out);
void cuboid_order(int T, int H, int W, int ct, int ch, int cw, int prefix, int32_t* out);

// Standard normal quantile (Wichura's algorithm AS 241, PPND16), p in (0, 1).
double normal_quantile(double p);

}  // namespace dbs
