// chunked.hip -- chunked prefill of the gated delta rule on gfx950 MFMA.
//
// Recurrence (per sequence and head; KDA: per-channel gate, GDN: scalar gate,
// "Super Apriel: One Checkpoint, Many Speeds", gist.science summary 2a):
//     S_t = S_{t-1} Diag(a_t)(I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
//     o_t = scale * S_t q_t.
//
// Chunked form used here (an exact reorganisation; derivation below).  For a
// chunk of C = 64 tokens starting from state S0 (Dv x Dk), with the
// in-chunk cumulative log gate b_r = sum_{s<=r} g_s (per channel for KDA,
// one scalar for GDN) and Gamma_r = exp(b_r):
//     Qt = q (.) e^{b},  Kt = k (.) e^{b},  Kb = k (.) e^{-b},
//     Kh = k (.) e^{b_C - b}                            (rows are tokens)
//     A  = strict_lower(Kt Kb^T),  P = lower(Qt Kb^T)     (C x C)
//     T  = (I + diag(beta) A)^{-1} diag(beta)             (UT transform)
//     X  = V - Kt S0^T,   U = T X                         (C x Dv)
//     O  = scale (Qt S0^T + P U)
//     S_C = S0 Diag(e^{b_C}) + U^T Kh
// Derivation: with u_r = beta_r (v_r - S'_{r} k_r) the recurrence is
// S_r = S_{r-1} Diag(a_r) + u_r k_r^T, so S_r = S0 Gamma_r
// + sum_{s<=r} u_s (k_s Gamma_s^{-1} Gamma_r)^T.  Substituting into u_r gives
// (I + diag(beta) A) U = diag(beta)(V - Kt S0^T); o_r = S_r q_r gives O; and
// S_C is the r = C case.  For GDN every exponential is a scalar per token,
// so A and P are scaled by e^{b_r - b_s} after the product instead.
//
// Work split.  One workgroup (4 waves) owns one (sequence, head, 32-wide
// slice of Dv) and walks its chunks in order; the Dv slices of a head are
// independent (rows of S never mix), which gives Dv/32 workgroups per head.
// The slices of one head are placed on one XCD so their shared reads of
// q, k and g hit the same L2.  All contractions use
// v_mfma_f32_16x16x32_bf16 (bf16 operands, fp32 accumulation); the state is
// carried between chunks in fp32 registers and rounded to bf16 only as an
// MFMA operand.  The UT transform inverts the four 16x16 diagonal blocks by
// forward substitution in fp32 and builds the off-diagonal blocks with
// 16x16x16 MFMAs (block forward substitution).
#include "gdr_internal.h"

namespace gdr {
namespace {

constexpr int C = 64;       // chunk length
constexpr int NW = 4;       // waves per workgroup
constexpr int BV = 32;      // value columns per workgroup
constexpr int PC = C + 8;   // padded LDS row length for C-wide bf16 rows
constexpr int PL = C + 4;   // padded LDS row length for the fp32 C x C matrix
constexpr int PV = BV + 8;  // padded LDS row length of the v tile
constexpr float kLog2e = 1.4426950408889634f;

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

template <int D, bool CH> struct Smem {
    static constexpr int PD = D + 8;   // padded row length for D-wide rows
    alignas(16) bf16 Q[C * PD];        // q (GDN) or q (.) e^b (KDA)
    alignas(16) bf16 K[C * PD];        // k (GDN) or k (.) e^b (KDA)
    alignas(16) bf16 Kb[CH ? C * PD : 8];   // k (.) e^-b (KDA)
    alignas(16) bf16 KhT[D * PC];      // (k (.) e^{b_C - b})^T
    alignas(16) bf16 S[BV * PD];       // state slice S0[i][j], bf16 copy
    alignas(16) bf16 Tm[C * PC];       // T
    alignas(16) bf16 P[C * PC];        // P
    alignas(16) bf16 XT[BV * PC];      // X^T
    alignas(16) bf16 UT[BV * PC];      // U^T
    alignas(16) bf16 V[C * PV];        // v tile
    alignas(16) float L[C * PL];       // diag(beta) A, then inverted diagonal blocks
    alignas(16) float gb[C];           // GDN: cumulative log gate per row
    alignas(16) float beta[C];
    alignas(16) float gam[D];          // e^{b_C} per channel (GDN: gam[0])
    alignas(16) float tot[NW * D];     // KDA: per-wave partial sums of g
};

template <int D, bool CH>
__global__ __launch_bounds__(256, 1) void chunked_kernel(PrefillArgs a) {
    using Sm = Smem<D, CH>;
    constexpr int PD = Sm::PD;
    constexpr int NTILE = D / BV;
    constexpr int CG = D / 8;          // 8-channel groups per row
    constexpr int RG = 256 / CG;       // row groups
    constexpr int RPT = C / RG;        // rows per thread in the gate phase
    constexpr int KD = D / 32;         // x32 steps over a D-long contraction
    constexpr int JKW = D / 16 / NW;   // 16-row blocks of S^T per wave
    __shared__ Sm sm;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = tid >> 6;
    const int l15 = lane & 15;
    const int l4 = lane >> 4;

    // ---- work mapping: the Dv slices of one (sequence, head) share an XCD
    const int bid = blockIdx.x;
    const int xcd = bid & 7;
    const int jj = bid >> 3;
    const int tile = jj % NTILE;
    const int unit = (jj / NTILE) * 8 + xcd;
    if (unit >= a.N * a.H) return;
    const int rank = unit / a.H;
    const int h = unit - rank * a.H;
    const int n = a.order ? a.order[rank] : rank;
    long long t0, t1;
    if (a.cu_seqlens) {
        t0 = a.cu_seqlens[n];
        t1 = a.cu_seqlens[n + 1];
    } else {
        t0 = (long long)n * a.T;
        t1 = t0 + a.T;
    }
    const int i0 = tile * BV;
    const size_t sslot = ((size_t)n * a.H + h) * D * D;
    const size_t tokstride = (size_t)a.H * D;
    const bf16 *qg = static_cast<const bf16 *>(a.q) + (size_t)h * D;
    const bf16 *kg = static_cast<const bf16 *>(a.k) + (size_t)h * D;
    const bf16 *vg = static_cast<const bf16 *>(a.v) + (size_t)h * D + i0;
    bf16 *og = static_cast<bf16 *>(a.o) + (size_t)h * D + i0;

    // T and P keep zero upper triangles: only lower blocks are ever written
    for (int e = tid; e < C * PC; e += 256) {
        sm.Tm[e] = (bf16)0.f;
        sm.P[e] = (bf16)0.f;
    }

    // ---- state S^T blocks in registers: lane holds S^T[j][iv] for
    //      j = 16*Jk + 4*l4 + e, iv = 16*Jv + l15, Jk = w*JKW + jk
    f32x4 St[JKW][2];
#pragma unroll
    for (int jk = 0; jk < JKW; ++jk) {
#pragma unroll
        for (int jv = 0; jv < 2; ++jv) {
            const int j = 16 * (w * JKW + jk) + 4 * l4;
            const int iv = 16 * jv + l15;
            f32x4 s = {0.f, 0.f, 0.f, 0.f};
            if (a.h0) s = *reinterpret_cast<const f32x4 *>(a.h0 + sslot + (size_t)(i0 + iv) * D + j);
            St[jk][jv] = s;
            *reinterpret_cast<bf16x4 *>(&sm.S[iv * PD + j]) = cvt4(s);
        }
    }

    const int cg = tid % CG;
    const int rg = tid / CG;
    const long long nchunks = (t1 - t0 + C - 1) / C;

    for (long long c = 0; c < nchunks; ++c) {
        const long long tc = t0 + c * C;
        const int Cc = (int)((t1 - tc) < C ? (t1 - tc) : C);

        // ================= phase 1a: load the chunk =====================
        bf16x8 q8[RPT], k8[RPT];
        float gsum[8];
        float cum[RPT][8];
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            const int r = rg * RPT + i;
            if (r < Cc) {
                const size_t off = (size_t)(tc + r) * tokstride + 8 * cg;
                q8[i] = ld8(qg + off);
                k8[i] = ld8(kg + off);
            } else {
                q8[i] = bf16x8{};
                k8[i] = bf16x8{};
            }
        }
        {   // v tile [C][BV]: 4 threads per row, 8 values each
            const int vr = tid / (BV / 8);
            const int vc = (tid % (BV / 8)) * 8;
            bf16x8 v8 = bf16x8{};
            if (vr < Cc) v8 = ld8(vg + (size_t)(tc + vr) * tokstride + vc);
            *reinterpret_cast<bf16x8 *>(&sm.V[vr * PV + vc]) = v8;
        }
        if (tid < C)
            sm.beta[tid] = tid < Cc ? a.beta[(size_t)(tc + tid) * a.H + h] : 0.f;
        if (CH) {
            // per-thread running sums over its RPT rows, 8 channels
#pragma unroll
            for (int e = 0; e < 8; ++e) gsum[e] = 0.f;
#pragma unroll
            for (int i = 0; i < RPT; ++i) {
                const int r = rg * RPT + i;
                f32x4 g0 = {0.f, 0.f, 0.f, 0.f}, g1 = {0.f, 0.f, 0.f, 0.f};
                if (r < Cc) {
                    const float *gp = a.g + ((size_t)(tc + r) * a.H + h) * D + 8 * cg;
                    g0 = *reinterpret_cast<const f32x4 *>(gp);
                    g1 = *reinterpret_cast<const f32x4 *>(gp + 4);
                }
                const float gv[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    gsum[e] += gv[e];
                    cum[i][e] = gsum[e];
                }
            }
            // inclusive scan of the row-group totals across the wave
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float incl = gsum[e];
#pragma unroll
                for (int off = CG; off < 64; off *= 2) {
                    const float y = __shfl_up(incl, off);
                    if (lane >= off) incl += y;
                }
                const float excl = incl - gsum[e];
#pragma unroll
                for (int i = 0; i < RPT; ++i) cum[i][e] += excl;
                if (lane >= 64 - CG) sm.tot[w * D + 8 * cg + e] = incl;
            }
        } else if (w == 0) {
            float gv = lane < Cc ? a.g[(size_t)(tc + lane) * a.H + h] : 0.f;
#pragma unroll
            for (int off = 1; off < 64; off *= 2) {
                const float y = __shfl_up(gv, off);
                if (lane >= off) gv += y;
            }
            sm.gb[lane] = gv;
        }
        __syncthreads();

        // ================= phase 1b: gated operands in LDS ================
        if (CH) {
            float bC[8], pre[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) { bC[e] = 0.f; pre[e] = 0.f; }
#pragma unroll
            for (int ww = 0; ww < NW; ++ww) {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float t = sm.tot[ww * D + 8 * cg + e];
                    bC[e] += t;
                    if (ww < w) pre[e] += t;
                }
            }
            float gC[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) gC[e] = ex(bC[e]);
            if (rg == 0) {
#pragma unroll
                for (int e = 0; e < 8; ++e) sm.gam[8 * cg + e] = gC[e];
            }
            float kh[RPT][8];
#pragma unroll
            for (int i = 0; i < RPT; ++i) {
                const int r = rg * RPT + i;
                float qt[8], kt[8], kb[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float eb = ex(cum[i][e] + pre[e]);
                    const float ebi = __builtin_amdgcn_rcpf(eb);
                    const float kv = (float)k8[i][e];
                    qt[e] = (float)q8[i][e] * eb;
                    kt[e] = kv * eb;
                    kb[e] = kv * ebi;
                    kh[i][e] = kb[e] * gC[e];
                }
                *reinterpret_cast<bf16x8 *>(&sm.Q[r * PD + 8 * cg]) = cvt8(qt);
                *reinterpret_cast<bf16x8 *>(&sm.K[r * PD + 8 * cg]) = cvt8(kt);
                *reinterpret_cast<bf16x8 *>(&sm.Kb[r * PD + 8 * cg]) = cvt8(kb);
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                bf16 *dst = &sm.KhT[(8 * cg + e) * PC + rg * RPT];
#pragma unroll
                for (int i = 0; i < RPT; ++i) dst[i] = (bf16)kh[i][e];
            }
        } else {
            const float bC = sm.gb[C - 1];
            if (tid == 0) sm.gam[0] = ex(bC);
#pragma unroll
            for (int i = 0; i < RPT; ++i) {
                const int r = rg * RPT + i;
                *reinterpret_cast<bf16x8 *>(&sm.Q[r * PD + 8 * cg]) = q8[i];
                *reinterpret_cast<bf16x8 *>(&sm.K[r * PD + 8 * cg]) = k8[i];
            }
            float sc[RPT];
#pragma unroll
            for (int i = 0; i < RPT; ++i) sc[i] = ex(bC - sm.gb[rg * RPT + i]);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                bf16 *dst = &sm.KhT[(8 * cg + e) * PC + rg * RPT];
#pragma unroll
                for (int i = 0; i < RPT; ++i) dst[i] = (bf16)((float)k8[i][e] * sc[i]);
            }
        }
        __syncthreads();

        // ================= phase 2: A, P, X, Qt S0^T on MFMA ===============
        const bf16 *Bop = CH ? sm.Kb : sm.K;
        for (int jb = w; jb < 20; jb += NW) {
            const bool isP = jb >= 10;
            const int tri = isP ? jb - 10 : jb;
            const int I = tri < 1 ? 0 : tri < 3 ? 1 : tri < 6 ? 2 : 3;
            const int J = tri - I * (I + 1) / 2;
            const bf16 *Aop = isP ? sm.Q : sm.K;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < KD; ++kk)
                acc = mfma32(ld8(&Aop[(16 * I + l15) * PD + 32 * kk + 8 * l4]),
                             ld8(&Bop[(16 * J + l15) * PD + 32 * kk + 8 * l4]), acc);
            const int s = 16 * J + l15;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * I + 4 * l4 + e;
                float val = acc[e];
                if (!CH) val *= ex(fminf(sm.gb[r] - sm.gb[s], 0.f));
                if (isP) {
                    sm.P[r * PC + s] = (bf16)(s <= r ? val : 0.f);
                } else {
                    sm.L[r * PL + s] = s < r ? val * sm.beta[r] : 0.f;
                }
            }
        }
        f32x4 accO[2];
#pragma unroll
        for (int jv = 0; jv < 2; ++jv) {
            f32x4 x = {0.f, 0.f, 0.f, 0.f};
            f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < KD; ++kk) {
                const bf16x8 sop = ld8(&sm.S[(16 * jv + l15) * PD + 32 * kk + 8 * l4]);
                x = mfma32(ld8(&sm.K[(16 * w + l15) * PD + 32 * kk + 8 * l4]), sop, x);
                o = mfma32(ld8(&sm.Q[(16 * w + l15) * PD + 32 * kk + 8 * l4]), sop, o);
            }
            const int iv = 16 * jv + l15;
            f32x4 xv;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * w + 4 * l4 + e;
                const float gr = CH ? 1.f : ex(sm.gb[r]);
                xv[e] = (float)sm.V[r * PV + iv] - gr * x[e];
                o[e] *= gr;
            }
            *reinterpret_cast<bf16x4 *>(&sm.XT[iv * PC + 16 * w + 4 * l4]) = cvt4(xv);
            accO[jv] = o;
        }
        __syncthreads();

        // ================= phase 3a: invert diagonal 16x16 blocks =========
        {
            const int cc = l15;
            const float *Lb = &sm.L[(16 * w) * PL + 16 * w];
            float y[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float acc = 0.f;
#pragma unroll
                for (int s = 0; s < r; ++s) acc += Lb[r * PL + s] * y[s];
                y[r] = r == cc ? 1.f : (r < cc ? 0.f : -acc);
            }
            // each wave overwrites only its own block, after reading it
            if (lane < 16) {
                const float bc = sm.beta[16 * w + cc];
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    sm.L[(16 * w + r) * PL + 16 * w + cc] = y[r];
                    sm.Tm[(16 * w + r) * PC + 16 * w + cc] = (bf16)(y[r] * bc);
                }
            }
        }
        __syncthreads();

        // ================= phase 3b: off-diagonal blocks of T =============
        if (w == 0) {
            // A operand: fp32 block (bi, bk) of sm.L, row l15, cols 4*l4..+3
            auto opA = [&](int bi, int bk) -> bf16x4 {
                return cvt4(*reinterpret_cast<const f32x4 *>(&sm.L[(16 * bi + l15) * PL + 16 * bk + 4 * l4]));
            };
            // B operand: block (bk, bj), rows 4*l4..+3, col l15
            auto opB = [&](int bk, int bj) -> bf16x4 {
                const float *p = &sm.L[(16 * bk + 4 * l4) * PL + 16 * bj + l15];
                return bf16x4{(bf16)p[0], (bf16)p[PL], (bf16)p[2 * PL], (bf16)p[3 * PL]};
            };
            const f32x4 z0 = {0.f, 0.f, 0.f, 0.f};
            // Y_ij = -Y_ii * sum_{k=j}^{i-1} L_ik Y_kj
            f32x4 Y10 = -mfma16(opA(1, 1), cvt4(mfma16(opA(1, 0), opB(0, 0), z0)), z0);
            f32x4 Y21 = -mfma16(opA(2, 2), cvt4(mfma16(opA(2, 1), opB(1, 1), z0)), z0);
            f32x4 Y32 = -mfma16(opA(3, 3), cvt4(mfma16(opA(3, 2), opB(2, 2), z0)), z0);
            f32x4 Y20 = -mfma16(opA(2, 2),
                                cvt4(mfma16(opA(2, 1), cvt4(Y10), mfma16(opA(2, 0), opB(0, 0), z0))), z0);
            f32x4 Y31 = -mfma16(opA(3, 3),
                                cvt4(mfma16(opA(3, 2), cvt4(Y21), mfma16(opA(3, 1), opB(1, 1), z0))), z0);
            f32x4 Y30 = -mfma16(opA(3, 3),
                                cvt4(mfma16(opA(3, 2), cvt4(Y20),
                                            mfma16(opA(3, 1), cvt4(Y10), mfma16(opA(3, 0), opB(0, 0), z0)))),
                                z0);
            auto put = [&](int bi, int bj, f32x4 y) {
                const int s = 16 * bj + l15;
                const float bs = sm.beta[s];
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    sm.Tm[(16 * bi + 4 * l4 + e) * PC + s] = (bf16)(y[e] * bs);
            };
            put(1, 0, Y10);
            put(2, 1, Y21);
            put(3, 2, Y32);
            put(2, 0, Y20);
            put(3, 1, Y31);
            put(3, 0, Y30);
        }
        __syncthreads();

        // ================= phase 4: U = T X ==============================
        const int nk = w < 2 ? 1 : 2;   // T is lower triangular
#pragma unroll
        for (int jv = 0; jv < 2; ++jv) {
            f32x4 u = {0.f, 0.f, 0.f, 0.f};
            for (int kk = 0; kk < nk; ++kk)
                u = mfma32(ld8(&sm.Tm[(16 * w + l15) * PC + 32 * kk + 8 * l4]),
                           ld8(&sm.XT[(16 * jv + l15) * PC + 32 * kk + 8 * l4]), u);
            *reinterpret_cast<bf16x4 *>(&sm.UT[(16 * jv + l15) * PC + 16 * w + 4 * l4]) = cvt4(u);
        }
        __syncthreads();

        // ================= phase 5: outputs and the next state ============
#pragma unroll
        for (int jv = 0; jv < 2; ++jv) {
            f32x4 o = accO[jv];
            for (int kk = 0; kk < nk; ++kk)
                o = mfma32(ld8(&sm.P[(16 * w + l15) * PC + 32 * kk + 8 * l4]),
                           ld8(&sm.UT[(16 * jv + l15) * PC + 32 * kk + 8 * l4]), o);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * w + 4 * l4 + e;
                if (r < Cc) og[(size_t)(tc + r) * tokstride + 16 * jv + l15] = (bf16)(a.scale * o[e]);
            }
        }
#pragma unroll
        for (int jk = 0; jk < JKW; ++jk) {
            const int Jk = w * JKW + jk;
            const int j = 16 * Jk + 4 * l4;
            f32x4 gm;
            if (CH) gm = *reinterpret_cast<const f32x4 *>(&sm.gam[j]);
            else    gm = f32x4{sm.gam[0], sm.gam[0], sm.gam[0], sm.gam[0]};
#pragma unroll
            for (int jv = 0; jv < 2; ++jv) {
                f32x4 s = St[jk][jv] * gm;
#pragma unroll
                for (int kk = 0; kk < C / 32; ++kk)
                    s = mfma32(ld8(&sm.KhT[(16 * Jk + l15) * PC + 32 * kk + 8 * l4]),
                               ld8(&sm.UT[(16 * jv + l15) * PC + 32 * kk + 8 * l4]), s);
                St[jk][jv] = s;
                *reinterpret_cast<bf16x4 *>(&sm.S[(16 * jv + l15) * PD + j]) = cvt4(s);
            }
        }
    }

    if (a.ht) {
#pragma unroll
        for (int jk = 0; jk < JKW; ++jk) {
#pragma unroll
            for (int jv = 0; jv < 2; ++jv) {
                const int j = 16 * (w * JKW + jk) + 4 * l4;
                const int iv = 16 * jv + l15;
                *reinterpret_cast<f32x4 *>(a.ht + sslot + (size_t)(i0 + iv) * D + j) = St[jk][jv];
            }
        }
    }
}

// Longest sequence first: rank = number of sequences that are longer, or
// equally long with a smaller index (a stable descending order).
__global__ __launch_bounds__(256) void schedule_kernel(const int32_t *cu, int N, int32_t *order) {
    const int n = blockIdx.x * 256 + threadIdx.x;
    if (n >= N) return;
    const int len = cu[n + 1] - cu[n];
    int rank = 0;
    for (int m = 0; m < N; ++m) {
        const int lm = cu[m + 1] - cu[m];
        rank += (lm > len) || (lm == len && m < n);
    }
    order[rank] = n;
}

}  // namespace

hipError_t launch_prefill_chunked(int D, const PrefillArgs &a, hipStream_t s) {
    const long long units = (long long)a.N * a.H;
    if (units <= 0) return hipSuccess;
    const int ntile = D / BV;
    const long long blocks = ((units + 7) / 8) * 8 * ntile;
    dim3 grid((unsigned)blocks), block(256);
    if (D == 128) {
        if (a.channel_gate) hipLaunchKernelGGL((chunked_kernel<128, true>), grid, block, 0, s, a);
        else                hipLaunchKernelGGL((chunked_kernel<128, false>), grid, block, 0, s, a);
    } else {
        if (a.channel_gate) hipLaunchKernelGGL((chunked_kernel<64, true>), grid, block, 0, s, a);
        else                hipLaunchKernelGGL((chunked_kernel<64, false>), grid, block, 0, s, a);
    }
    return hipGetLastError();
}

hipError_t launch_varlen_schedule(const int32_t *cu_seqlens, int N, int32_t *order,
                                  hipStream_t s) {
    if (N <= 0) return hipSuccess;
    dim3 grid((unsigned)((N + 255) / 256)), block(256);
    hipLaunchKernelGGL(schedule_kernel, grid, block, 0, s, cu_seqlens, N, order);
    return hipGetLastError();
}

}  // namespace gdr
