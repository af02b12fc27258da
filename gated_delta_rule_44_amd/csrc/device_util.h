// device_util.h -- small device helpers shared by the chunked prefill
// kernels: MFMA wrappers, operand fragment loads from LDS, DPP broadcast and
// bounds-checked buffer accesses.  gfx950 only.
#pragma once

#include <type_traits>

#include "gdr_internal.h"

namespace gdr {

constexpr float kLog2e = 1.4426950408889634f;

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

__device__ inline float ex(float x) { return __builtin_amdgcn_exp2f(x * kLog2e); }

__device__ inline f32x4 mfma32(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ inline f32x4 mfma16(bf16x4 a, bf16x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
__device__ inline bf16x8 ld8(const bf16 *p) { return *reinterpret_cast<const bf16x8 *>(p); }
__device__ inline bf16x4 cvt4(f32x4 x) {
    return bf16x4{(bf16)x.x, (bf16)x.y, (bf16)x.z, (bf16)x.w};
}
__device__ inline bf16x8 cvt8(const float *x) {
    return bf16x8{(bf16)x[0], (bf16)x[1], (bf16)x[2], (bf16)x[3],
                  (bf16)x[4], (bf16)x[5], (bf16)x[6], (bf16)x[7]};
}

// MFMA fragment of a row-major [rows][ld] bf16 tile: lane holds row
// r0 + (lane & 15), columns k0 + 8 * (lane >> 4) .. +7.  This is the A operand
// of A(rows) x B, and the B operand of X Y^T with Y row-major.
__device__ inline bf16x8 frag_rows(const bf16 *base, int ld, int r0, int k0, int lane) {
    return ld8(base + (r0 + (lane & 15)) * ld + k0 + 8 * (lane >> 4));
}

// MFMA fragment read across rows of a row-major [k][ld] bf16 tile: lane
// holds column n0 + (lane & 15), rows k0 + 8 * (lane >> 4) .. +7.  Built from
// two ds_read_b64_tr_b16: within each 16-lane group, output lane i, slot m
// receives element (i & 3) of the 4-element segment addressed by lane
// (i >> 2) + 4m; addressing row (j >> 2), columns 4 (j & 3) from lane j
// therefore delivers rows 0..3 of column i to lane i.
__device__ inline bf16x8 frag_cols(const bf16 *base, int ld, int k0, int n0, int lane) {
    const int i = lane & 15;
    const bf16 *p = base + (k0 + 8 * (lane >> 4) + (i >> 2)) * ld + n0 + 4 * (i & 3);
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(p));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(p + 4 * ld));
    typedef short s16x8 __attribute__((ext_vector_type(8)));
    const s16x8 v = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
    return __builtin_bit_cast(bf16x8, v);
}

// x from lane q of each quad of lanes (DPP quad_perm broadcast).
__device__ inline float quad_bcast(float x, int q) {
    const int v = __builtin_bit_cast(int, x);
    int r;
    switch (q) {
    case 0: r = __builtin_amdgcn_mov_dpp(v, 0x00, 0xF, 0xF, false); break;
    case 1: r = __builtin_amdgcn_mov_dpp(v, 0x55, 0xF, 0xF, false); break;
    case 2: r = __builtin_amdgcn_mov_dpp(v, 0xAA, 0xF, 0xF, false); break;
    default: r = __builtin_amdgcn_mov_dpp(v, 0xFF, 0xF, 0xF, false); break;
    }
    return __builtin_bit_cast(float, r);
}

// Bounds-checked buffer accesses: a load past nbytes returns zeros and a
// store past it is dropped, so ragged chunk tails and absent chunks need no
// branches and every path issues the same memory operations (which keeps the
// compiler's wait counts exact for loads issued a chunk ahead).
typedef __amdgpu_buffer_rsrc_t rsrc_t;
// Every argument is wave-uniform at each call site; readfirstlane states it
// so the descriptor lives in scalar registers (a descriptor in vector
// registers would make the compiler loop over its distinct values).
__device__ inline rsrc_t make_rsrc(const void *base, unsigned nbytes) {
    const unsigned long long p = reinterpret_cast<unsigned long long>(base);
    const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)p);
    const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)(p >> 32));
    void *ub = reinterpret_cast<void *>(((unsigned long long)hi << 32) | lo);
    return __builtin_amdgcn_make_buffer_rsrc(ub, (short)0,
                                             (int)__builtin_amdgcn_readfirstlane(nbytes),
                                             0x00020000);
}
__device__ inline bf16x8 bload16(rsrc_t r, unsigned off) {
    return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ inline f32x4 bload16f(rsrc_t r, unsigned off) {
    return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ inline bf16x4 bload8(rsrc_t r, unsigned off) {
    return __builtin_bit_cast(bf16x4, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
}
__device__ inline float bload4(rsrc_t r, unsigned off) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}
__device__ inline void bstore2(rsrc_t r, unsigned off, bf16 v) {
    __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, v), r, off, 0, 0);
}
__device__ inline void bstore8s(rsrc_t r, unsigned voff, unsigned soff, bf16x4 v) {
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(__attribute__((ext_vector_type(2))) unsigned, v),
                                          r, voff, (int)__builtin_amdgcn_readfirstlane(soff), 0);
}
__device__ inline void bstore16s(rsrc_t r, unsigned voff, unsigned soff, bf16x8 v) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned, v),
                                           r, voff, (int)__builtin_amdgcn_readfirstlane(soff), 0);
}
// same with a wave-uniform part of the offset in a scalar register
__device__ inline void bstore2s(rsrc_t r, unsigned voff, unsigned soff, bf16 v) {
    __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, v), r, voff,
                                          (int)__builtin_amdgcn_readfirstlane(soff), 0);
}

// Inclusive prefix sum over the 64 lanes of a wave with DPP: shifts by 1, 2,
// 4, 8 within each row of 16 lanes (a lane whose source lies before its row
// adds 0), then the last lane of row 0 into row 1 and of row 2 into row 3
// (row_bcast:15), then the last lane of row 1 into rows 2 and 3
// (row_bcast:31).
__device__ inline float wave_prefix_sum(float v) {
    auto shr = [](float x, auto ctrl) -> float {
        return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x),
                                                                     decltype(ctrl)::value, 0xF, 0xF, true));
    };
    v += shr(v, std::integral_constant<int, 0x111>{});   // row_shr:1
    v += shr(v, std::integral_constant<int, 0x112>{});   // row_shr:2
    v += shr(v, std::integral_constant<int, 0x114>{});   // row_shr:4
    v += shr(v, std::integral_constant<int, 0x118>{});   // row_shr:8
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x142, 0xA, 0xF, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x143, 0xC, 0xF, false));
    return v;
}

// A copy of x the compiler cannot see through: lane-dependent addresses are
// rebuilt from it each iteration instead of being hoisted out of the chunk
// loop (where they would occupy registers for the whole loop).
__device__ inline int opaque(int x) {
    int y;
    asm volatile("v_mov_b32 %0, %1" : "=v"(y) : "v"(x));
    return y;
}


// Operand fragments in "paired" k order.  A 16x16x32 MFMA sums over 32 k
// slots; lane l supplies slots 8(l>>4)..+7.  When the other operand comes
// straight from two 16x16 accumulator blocks (lane l holds rows 4(l>>4)..+3
// of each), slot 8(l>>4)+u stands for k = k0 + 4(l>>4) + u for u < 4 and
// k = k0 + 16 + 4(l>>4) + (u-4) for u >= 4.  Any consistent k order gives the
// same sum.
__device__ inline bf16x8 cat8(bf16x4 lo, bf16x4 hi) {
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}
// B (or A) operand from two accumulator blocks: rows 4(l>>4)+e of x0 then x1.
__device__ inline bf16x8 acc_pair(f32x4 x0, f32x4 x1) { return cat8(cvt4(x0), cvt4(x1)); }
// Row r0 + (l & 15) of a row-major [rows][ld] bf16 tile, paired k order.
__device__ inline bf16x8 frag_pair_rows(const bf16 *base, int ld, int r0, int k0, int lane) {
    const bf16 *p = base + (r0 + (lane & 15)) * ld + k0 + 4 * (lane >> 4);
    return cat8(*reinterpret_cast<const bf16x4 *>(p), *reinterpret_cast<const bf16x4 *>(p + 16));
}
// Column n0 + (l & 15) of a row-major [k][ld] bf16 tile, paired k order, from
// two ds_read_b64_tr_b16 (see frag_cols): lane j of each 16-lane group
// addresses row k0 + 4(l>>4) + (j >> 2), columns n0 + 4(j & 3).
__device__ inline bf16x8 frag_pair_cols(const bf16 *base, int ld, int k0, int n0, int lane) {
    const int i = lane & 15;
    const bf16 *p = base + (k0 + 4 * (lane >> 4) + (i >> 2)) * ld + n0 + 4 * (i & 3);
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(p));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(p + 16 * ld));
    return cat8(__builtin_bit_cast(bf16x4, lo), __builtin_bit_cast(bf16x4, hi));
}
// Rows k0 + 4(l>>4) .. +3 of column n0 + (l & 15) of a row-major [k][ld] bf16
// tile, i.e. a 16x16 block of it in accumulator order, by one transpose load.
__device__ inline bf16x4 frag_col4(const bf16 *base, int ld, int k0, int n0, int lane) {
    const int i = lane & 15;
    const bf16 *p = base + (k0 + 4 * (lane >> 4) + (i >> 2)) * ld + n0 + 4 * (i & 3);
    return __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(p)));
}
// A 16x16 block kept in LDS in accumulator order: 256 bf16, lane l's four
// values (rows 4(l>>4)+e, column l&15) at 4l.  Stored and read back by the
// lane that owns them, so reads are one conflict-free ds_read_b64.
__device__ inline bf16x4 tile_ld(const bf16 *t, int lane) {
    return *reinterpret_cast<const bf16x4 *>(t + 4 * lane);
}
__device__ inline void tile_st(bf16 *t, int lane, f32x4 v) {
    *reinterpret_cast<bf16x4 *>(t + 4 * lane) = cvt4(v);
}
__device__ inline f32x4 mfma32z(bf16x8 a, bf16x8 b) {
    return mfma32(a, b, f32x4{0.f, 0.f, 0.f, 0.f});
}
__device__ inline f32x4 mfma16z(bf16x4 a, bf16x4 b) {
    return mfma16(a, b, f32x4{0.f, 0.f, 0.f, 0.f});
}
// Cross-lane sums on the VALU (no LDS round trip, so no wait on other LDS
// traffic in flight).  DPP within a 16-lane row; the gfx950 swaps across
// rows: v_permlane16_swap exchanges odd rows of one register with even rows
// of the other, v_permlane32_swap the upper half of one with the lower half
// of the other, so with both registers holding x, their sum is
// x[l] + x[l ^ 16] (resp. x[l ^ 32]) in every lane.  (Written out in asm:
// both registers of a swap carry a result; s_nop 1 covers the VALU write ->
// permlane read hazard.)
template <int CTRL>
__device__ inline float dpp_f(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                                 CTRL, 0xF, 0xF, true));
}
__device__ inline float swap_sum16(float x) {
    float a = x, b = x;
    asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(a), "+v"(b));
    return a + b;
}
__device__ inline float swap_sum32(float x) {
    float a = x, b = x;
    asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
    return a + b;
}
// sum over the lanes of the wave congruent to this one modulo S (S = 4 or 8)
template <int S>
__device__ inline float sum_stride(float x) {
    static_assert(S == 4 || S == 8, "stride");
    x += dpp_f<0x128>(x);                   // row_ror:8
    if (S == 4) x += dpp_f<0x124>(x);       // row_ror:4
    return swap_sum32(swap_sum16(x));
}
// sum over each aligned group of G consecutive lanes (G = 8 or 16)
template <int G>
__device__ inline float sum_group(float x) {
    static_assert(G == 8 || G == 16, "group");
    x += dpp_f<0xB1>(x);                    // quad_perm [1,0,3,2]
    x += dpp_f<0x4E>(x);                    // quad_perm [2,3,0,1]
    x += dpp_f<0x141>(x);                   // row_half_mirror
    if (G == 16) x += dpp_f<0x140>(x);      // row_mirror
    return x;
}

__device__ inline float bf16_bits_to_float(unsigned short h) {
    return __builtin_bit_cast(float, (unsigned)h << 16);
}
__device__ inline unsigned short bload2(rsrc_t r, unsigned off) {
    return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
}

}  // namespace gdr
