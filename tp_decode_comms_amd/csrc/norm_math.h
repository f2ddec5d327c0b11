// norm_math.h -- fixed-order arithmetic of the residual add + RMS norm that
// follows the AllReduce in a decode layer ("vLLM 分布式推理核心" page,
// sections 一 and 二: once the AllReduce completes the compute stream goes on
// with the layer's norm).  The page names the op without defining it; the
// form computed here is the residual add followed by the weighted RMS norm:
//
//   h[i] = bf16( f32(a[i]) + f32(res[i]) )            a = AllReduce result
//   y[i] = bf16( (f32(h[i]) * r) * f32(gamma[i]) ),   r = 1 / sqrt(S/hidden + eps)
//
// with S the binary32 sum of h[j]^2 over the row.  S is always formed in one
// order, whichever kernel computes it: per 256-element block (64 lanes x 4
// consecutive elements), each lane sums its 4 squares left to right with
// fused multiply-adds, then the 64 lane sums meet in the fixed tree of
// wave_sum(); the row's block sums are then folded the same way, lane l
// holding blocks l, l+64, l+128, ... added in that order.  Both
// the fused kernel (each workgroup round yields one block's sum; the sums
// meet through memory) and the stand-alone kernel (one workgroup per row,
// block sums in LDS) follow it, so their h and y agree bit for bit.
#pragma once
#include "ar_kernels.h"
#include "ar_proto.h"

namespace ar {

constexpr uint32_t NORM_BLOCK = (uint32_t)NORM_BLOCK_ELEMS;        // elements per partial sum
constexpr uint32_t NORM_MAX_HIDDEN = (uint32_t)NORM_HIDDEN_LIMIT;
constexpr uint32_t NORM_MAX_BLOCKS = NORM_MAX_HIDDEN / NORM_BLOCK;

// h = bf16(a + res) for 4 elements (2 packed words each), one binary32
// addition per element rounded once to nearest even.
__device__ __forceinline__ u32x2 add_round4(u32x2 a, u32x2 r)
{
    u32x2 h;
    h.x = pack_bf16(lo_f(a.x) + lo_f(r.x), hi_f(a.x) + hi_f(r.x));
    h.y = pack_bf16(lo_f(a.y) + lo_f(r.y), hi_f(a.y) + hi_f(r.y));
    return h;
}

// sum of the squares of 4 bf16 values, left to right (explicit fused
// multiply-adds: the association is not left to the compiler)
__device__ __forceinline__ float sumsq4(u32x2 h)
{
    const float a = lo_f(h.x), b = hi_f(h.x), c = lo_f(h.y), d = hi_f(h.y);
    float s = a * a;
    s = __builtin_fmaf(b, b, s);
    s = __builtin_fmaf(c, c, s);
    s = __builtin_fmaf(d, d, s);
    return s;
}

// Wave-wide sum in a fixed tree.  Within each 16-lane row four DPP steps
// pair lane i with i^1, i^2 (quad permutes), then the mirror lane of its
// 8-lane half and of its row; binary32 addition commutes, so both lanes of
// every pair compute the same bits and the whole row ends with one value.
// The four row sums are then read as uniform values and added as
// (r0 + r1) + (r2 + r3), so all 64 lanes return identical bits.
template <int CTRL> __device__ __forceinline__ float dpp(float v)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}

__device__ __forceinline__ float wave_sum(float v)
{
    v += dpp<0xB1>(v);          // quad_perm(1,0,3,2): lane i ^ 1
    v += dpp<0x4E>(v);          // quad_perm(2,3,0,1): lane i ^ 2
    v += dpp<0x141>(v);         // row_half_mirror: lane 7 - i within 8
    v += dpp<0x140>(v);         // row_mirror: lane 15 - i within 16
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
    return (r0 + r1) + (r2 + r3);
}

// r = 1 / sqrt(S / hidden + eps): IEEE division and square root
__device__ __forceinline__ float rms_inv(float S, uint32_t hidden, float eps)
{
    const float mean = S / (float)hidden;
    return 1.0f / __builtin_sqrtf(mean + eps);
}

// y = bf16((h * r) * gamma) for 4 elements
__device__ __forceinline__ u32x2 scale4(u32x2 h, u32x2 g, float r)
{
    u32x2 y;
    const float t0 = lo_f(h.x) * r, t1 = hi_f(h.x) * r, t2 = lo_f(h.y) * r, t3 = hi_f(h.y) * r;
    y.x = pack_bf16(t0 * lo_f(g.x), t1 * hi_f(g.x));
    y.y = pack_bf16(t2 * lo_f(g.y), t3 * hi_f(g.y));
    return y;
}

}  // namespace ar
