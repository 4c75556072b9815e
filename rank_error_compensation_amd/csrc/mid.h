// Launcher of the 17 .. 64-token tile (prefill.hip, mid_kernel), internal.
#pragma once

#include "glowq_internal.h"

namespace glowq {

// One correcting launch over one token block: a.m_tiles == 1, a.tile_tt token tiles of 16 (2 or 4,
// covering T), a.tile_rr == 8 row tiles per workgroup, a.n_tiles row blocks numbered per module from
// mod[i].tile_begin, INT4 weights, a.r > 0; the launch forms the projection itself: a.n_prod
// producer workgroups first, R handed over as tagged pairs at a.R.
hipError_t launch_mid(const ForwardArgs& a, hipStream_t stream);

}  // namespace glowq
