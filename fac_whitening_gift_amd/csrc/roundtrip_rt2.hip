// The round-trip kernels with 32-row tiles (two 16-row MFMA tiles per
// workgroup, namespace gift::rt2): with half the rows per workgroup a small
// group has twice the workgroups, which shortens the last round of
// workgroups on the machine; the host side picks it for groups below 2^25
// whitened gradient elements.
#define GIFT_TILE_RT 2
#define GIFT_TILE_NS rt2
#include "roundtrip.hip"
