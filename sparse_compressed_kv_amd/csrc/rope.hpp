// rope.hpp — the tail RoPE angle and rotation shared by the attention kernel (the query)
// and the compressor (emitted rows), so that both rotate by the same bits.
//
// "Reading the architecture of DwarfStar (ds4.c), part 1/8" (Qiita), sections 2 and 3-2:
// RoPE acts on the last n_rot = 64 of the 512 dims; compressed rows are rotated when they
// are emitted.  Pairs are adjacent (D-n_rot+2i, D-n_rot+2i+1); the angle of pair i is
// pos * theta^(-2i/n_rot).
#pragma once

#include "common.hpp"

namespace ds4a {

namespace {

// The angle of the adjacent pair i of the tail, pos * theta^(-2i/n_rot), as (cos, sin)
// in fp64.  The angle (up to ~1e6 rad) is first reduced by a two-part 2*pi in fp64, so that
// sincos runs on |x| <= pi.
__device__ __forceinline__ void rope_angle(double log2_theta, int i, int64_t pos, double &cs, double &sn,
                                           int n_rot = 64) {
    const double inv_freq = exp2(-(double)(2 * i) / (double)n_rot * log2_theta);
    const double ang = (double)pos * inv_freq;
    const double k = rint(ang * 0.15915494309189535);          // 1 / (2 pi)
    double red = fma(-k, 6.283185307179586, ang);              // 2 pi, high part
    red = fma(-k, 2.4492935982947064e-16, red);                // 2 pi, low part
    sincos(red, &sn, &cs);
}

// Rotate the pair (a, b) by the angle (cs, sn) in fp64 and round once to f32.
__device__ __forceinline__ void rope_rotate(double cs, double sn, float &a, float &b) {
    const double x = (double)a, y = (double)b;
    a = (float)(x * cs - y * sn);
    b = (float)(x * sn + y * cs);
}

__device__ __forceinline__ void rope_pair(double log2_theta, int i, int64_t pos, float &a, float &b) {
    double cs, sn;
    rope_angle(log2_theta, i, pos, cs, sn);
    rope_rotate(cs, sn, a, b);
}

}  // namespace

}  // namespace ds4a
