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
// one scalar for GDN):
//     Qt = q (.) e^{b},  Kt = k (.) e^{b},  Kb = k (.) e^{-b},
//     Kh = k (.) e^{b_C - b}                            (rows are tokens)
//     A  = strict_lower(Kt Kb^T),  P = lower(Qt Kb^T)     (C x C)
//     T  = (I + diag(beta) A)^{-1} diag(beta)             (UT transform)
//     X  = V - Kt S0^T,   U = T X                         (C x Dv)
//     O  = scale (Qt S0^T + P U)
//     S_C = S0 Diag(e^{b_C}) + U^T Kh
// Derivation: with u_r = beta_r (v_r - S_{r-1} Diag(a_r) k_r) the recurrence
// is S_r = S_{r-1} Diag(a_r) + u_r k_r^T, so S_r = S0 Gamma_r
// + sum_{s<=r} u_s (k_s (.) e^{b_r - b_s})^T with Gamma_r = Diag(e^{b_r}).
// Substituting into u_r gives (I + diag(beta) A) U = diag(beta)(V - Kt S0^T);
// o_r = S_r q_r gives O; S_C is the r = C case.  For GDN every exponential is
// one scalar per token, so A and P are scaled by e^{b_r - b_s} after the
// product and Kt, Qt are row scalings applied to the products.
//
// Work split.  One workgroup (8 waves) owns one (sequence, head, 32-wide
// slice of Dv) and walks its chunks in order; rows of S never mix, so the
// Dv slices of a head are independent.  The slices of one head run on one
// XCD so their shared reads of q, k and g hit the same L2.  Each chunk:
//   1  gate prefix sums and gated operands -> LDS (next chunk's global
//      loads are issued right after, into registers)
//   2  A (for L = diag(beta) A), X = V - Kt S0^T and Qt S0^T on MFMA
//   3  wave 0: T = (I + L)^{-1} diag(beta): the four 16x16 diagonal blocks by
//      forward substitution in fp32, the others by 16x16x16 MFMA block
//      substitution; waves 1-7 meanwhile form P on MFMA
//   4  U = T X
//   5  O = Qt S0^T + P U, and S^T <- e^{b_C} (.) S^T + Kh^T U
// All contractions use bf16 operands with fp32 accumulation; the state is
// carried in fp32 registers and rounded to bf16 only as an MFMA operand.
#include "gdr_internal.h"

namespace gdr {
namespace {

constexpr int C = 64;       // chunk length
constexpr int NW = 8;       // waves per workgroup
constexpr int NT = NW * 64; // threads per workgroup
constexpr int BV = 32;      // value columns per workgroup
constexpr int PC = C + 8;   // padded LDS row length for C-wide bf16 rows
constexpr int PL = C + 4;   // padded LDS row length of the fp32 L^T
constexpr int PY = 20;      // padded row length of the fp32 16x16 blocks
constexpr int PV = BV + 8;  // padded LDS row length of the v tile
constexpr float kLog2e = 1.4426950408889634f;

typedef short s16x4 __attribute__((ext_vector_type(4)));

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
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(p));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(p + 4 * ld));
    typedef short s16x8 __attribute__((ext_vector_type(8)));
    const s16x8 v = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
    return __builtin_bit_cast(bf16x8, v);
}

template <int D, bool CH> struct Smem {
    static constexpr int PD = D + 8;   // padded row length for D-wide rows
    alignas(16) bf16 Q[C * PD];        // q (GDN) or q (.) e^b (KDA), [r][j]
    alignas(16) bf16 K[C * PD];        // k (GDN) or k (.) e^b (KDA), [r][j]
    alignas(16) bf16 Kb[CH ? C * PD : 8];   // k (.) e^-b (KDA), [r][j]
    alignas(16) bf16 Kh[C * PD];       // k (.) e^{b_C - b}, [s][j]
    alignas(16) bf16 S[BV * PD];       // bf16 copy of the state slice, [i][j]
    alignas(16) bf16 Tm[C * PC];       // T, [r][s]
    alignas(16) bf16 P[C * PC];        // P, [r][s]
    alignas(16) bf16 XT[BV * PC];      // X^T, [i][s]
    alignas(16) bf16 UT[BV * PC];      // U^T, [i][s]
    alignas(16) bf16 V[C * PV];        // v tile, [r][i]
    alignas(16) float LT[C * PL];      // L^T = (diag(beta) A)^T, [s][r]
    alignas(16) float Y[4 * 16 * PY];  // inverted diagonal blocks, [b][r][c]
    alignas(16) float gb[C];           // GDN: cumulative log gate per row
    alignas(16) float beta[C];
    alignas(16) float gam[D];          // e^{b_C} per channel (GDN: gam[0])
    alignas(16) float tot[NW * D];     // KDA: per-wave sums of g
};

template <int D, bool CH>
__global__ __launch_bounds__(NT, 1) void chunked_kernel(PrefillArgs a) {
    using Sm = Smem<D, CH>;
    constexpr int PD = Sm::PD;
    constexpr int NTILE = D / BV;
    constexpr int CG = D / 8;          // 8-channel groups per row
    constexpr int RPW = 64 / CG;       // row groups per wave
    constexpr int RPT = C / (NW * RPW);// rows per thread in the gate phase
    constexpr int KD = D / 32;         // x32 steps over a D-long contraction
    constexpr int SB = D / 64;         // S^T blocks per wave (x2 value blocks / NW)
    static_assert(RPT >= 1, "gate phase layout");
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
    for (int e = tid; e < C * PC; e += NT) {
        sm.Tm[e] = (bf16)0.f;
        sm.P[e] = (bf16)0.f;
    }

    // ---- state S^T blocks in registers: wave w, block sb holds S^T[j][iv]
    //      for j = 16*Jk + 4*l4 + e, iv = 16*Jv + l15
    auto jk_of = [&](int sb) { return SB == 2 ? w : (w >> 1); };
    auto jv_of = [&](int sb) { return SB == 2 ? sb : (w & 1); };
    f32x4 St[SB];
#pragma unroll
    for (int sb = 0; sb < SB; ++sb) {
        const int j = 16 * jk_of(sb) + 4 * l4;
        const int iv = 16 * jv_of(sb) + l15;
        f32x4 s = {0.f, 0.f, 0.f, 0.f};
        if (a.h0) s = *reinterpret_cast<const f32x4 *>(a.h0 + sslot + (size_t)(i0 + iv) * D + j);
        St[sb] = s;
        *reinterpret_cast<bf16x4 *>(&sm.S[iv * PD + j]) = cvt4(s);
    }

    // ---- gate-phase thread layout: 8 channels x RPT rows per thread
    const int cg = lane % CG;
    const int rg = w * RPW + lane / CG;
    const int vr = tid >> 3;              // v tile: 8 threads per row, 4 values each
    const int vc = (tid & 7) * 4;

    // ---- prefetch registers for one chunk
    bf16x8 q8[RPT], k8[RPT];
    f32x4 g8[CH ? RPT : 1][2];
    bf16x4 v4;
    float gsc = 0.f, bet = 0.f;
    auto prefetch = [&](long long tc, int Cc) {
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            const int r = rg * RPT + i;
            if (r < Cc) {
                const size_t off = (size_t)(tc + r) * tokstride + 8 * cg;
                q8[i] = ld8(qg + off);
                k8[i] = ld8(kg + off);
                if (CH) {
                    const float *gp = a.g + ((size_t)(tc + r) * a.H + h) * D + 8 * cg;
                    g8[i][0] = *reinterpret_cast<const f32x4 *>(gp);
                    g8[i][1] = *reinterpret_cast<const f32x4 *>(gp + 4);
                }
            } else {
                q8[i] = bf16x8{};
                k8[i] = bf16x8{};
                if (CH) {
                    g8[i][0] = f32x4{0.f, 0.f, 0.f, 0.f};
                    g8[i][1] = f32x4{0.f, 0.f, 0.f, 0.f};
                }
            }
        }
        v4 = vr < Cc ? *reinterpret_cast<const bf16x4 *>(vg + (size_t)(tc + vr) * tokstride + vc)
                     : bf16x4{};
        if (tid < C) {
            bet = tid < Cc ? a.beta[(size_t)(tc + tid) * a.H + h] : 0.f;
            if (!CH) gsc = tid < Cc ? a.g[(size_t)(tc + tid) * a.H + h] : 0.f;
        }
    };

    const long long nchunks = (t1 - t0 + C - 1) / C;
    if (nchunks > 0) prefetch(t0, (int)((t1 - t0) < C ? (t1 - t0) : C));

    for (long long c = 0; c < nchunks; ++c) {
        const long long tc = t0 + c * C;
        const int Cc = (int)((t1 - tc) < C ? (t1 - tc) : C);

        // ================= 1a: stage v and beta; gate prefix sums ==========
        *reinterpret_cast<bf16x4 *>(&sm.V[vr * PV + vc]) = v4;
        if (tid < C) sm.beta[tid] = bet;
        float cum[CH ? RPT : 1][8];
        if (CH) {
            float run[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) run[e] = 0.f;
#pragma unroll
            for (int i = 0; i < RPT; ++i) {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    run[e] += g8[i][e >> 2][e & 3];
                    cum[i][e] = run[e];
                }
            }
            // inclusive scan of the row-group sums across the wave
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float incl = run[e];
#pragma unroll
                for (int off = CG; off < 64; off *= 2) {
                    const float y = __shfl_up(incl, off);
                    if (lane >= off) incl += y;
                }
#pragma unroll
                for (int i = 0; i < RPT; ++i) cum[i][e] += incl - run[e];
                if (lane >= 64 - CG) sm.tot[w * D + 8 * cg + e] = incl;
            }
        } else if (w == 0) {
            float gv = gsc;
#pragma unroll
            for (int off = 1; off < 64; off *= 2) {
                const float y = __shfl_up(gv, off);
                if (lane >= off) gv += y;
            }
            sm.gb[lane] = gv;
        }
        __syncthreads();

        // ================= 1b: gated operands in LDS ======================
        if (CH) {
            float bC[8], pre[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) { bC[e] = 0.f; pre[e] = 0.f; }
#pragma unroll
            for (int ww = 0; ww < NW; ++ww) {
                const f32x4 t0v = *reinterpret_cast<const f32x4 *>(&sm.tot[ww * D + 8 * cg]);
                const f32x4 t1v = *reinterpret_cast<const f32x4 *>(&sm.tot[ww * D + 8 * cg + 4]);
                const float tv[8] = {t0v.x, t0v.y, t0v.z, t0v.w, t1v.x, t1v.y, t1v.z, t1v.w};
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    bC[e] += tv[e];
                    pre[e] += ww < w ? tv[e] : 0.f;
                }
            }
            float gC[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) gC[e] = ex(bC[e]);
            if (rg == 0) {
                *reinterpret_cast<f32x4 *>(&sm.gam[8 * cg]) = f32x4{gC[0], gC[1], gC[2], gC[3]};
                *reinterpret_cast<f32x4 *>(&sm.gam[8 * cg + 4]) = f32x4{gC[4], gC[5], gC[6], gC[7]};
            }
#pragma unroll
            for (int i = 0; i < RPT; ++i) {
                const int r = rg * RPT + i;
                float qt[8], kt[8], kb[8], kh[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float eb = ex(cum[i][e] + pre[e]);
                    const float ebi = __builtin_amdgcn_rcpf(eb);
                    const float kv = (float)k8[i][e];
                    qt[e] = (float)q8[i][e] * eb;
                    kt[e] = kv * eb;
                    kb[e] = kv * ebi;
                    kh[e] = kb[e] * gC[e];
                }
                *reinterpret_cast<bf16x8 *>(&sm.Q[r * PD + 8 * cg]) = cvt8(qt);
                *reinterpret_cast<bf16x8 *>(&sm.K[r * PD + 8 * cg]) = cvt8(kt);
                *reinterpret_cast<bf16x8 *>(&sm.Kb[r * PD + 8 * cg]) = cvt8(kb);
                *reinterpret_cast<bf16x8 *>(&sm.Kh[r * PD + 8 * cg]) = cvt8(kh);
            }
        } else {
            const float bC = sm.gb[C - 1];
            if (tid == 0) sm.gam[0] = ex(bC);
#pragma unroll
            for (int i = 0; i < RPT; ++i) {
                const int r = rg * RPT + i;
                const float sc = ex(bC - sm.gb[r]);
                float kh[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) kh[e] = (float)k8[i][e] * sc;
                *reinterpret_cast<bf16x8 *>(&sm.Q[r * PD + 8 * cg]) = q8[i];
                *reinterpret_cast<bf16x8 *>(&sm.K[r * PD + 8 * cg]) = k8[i];
                *reinterpret_cast<bf16x8 *>(&sm.Kh[r * PD + 8 * cg]) = cvt8(kh);
            }
        }
        // the next chunk's global loads overlap with everything below
        if (c + 1 < nchunks) {
            const long long tn = tc + C;
            prefetch(tn, (int)((t1 - tn) < C ? (t1 - tn) : C));
        }
        __syncthreads();

        // ================= 2: A -> L^T, X, Qt S0^T ========================
        const bf16 *Bop = CH ? sm.Kb : sm.K;
        const int Iw = w >> 1;          // this wave's 16-row block of X, U, O
        const int Jw = w & 1;           // and its 16-column value block
        f32x4 accO;
        {
            // A jobs: lower blocks (I, J), J <= I, numbered 0..9; wave w takes
            // job w and, for w < 2, job 8 + w
            auto jobIJ = [](int tri, int &I, int &J) {
                I = tri < 1 ? 0 : tri < 3 ? 1 : tri < 6 ? 2 : 3;
                J = tri - I * (I + 1) / 2;
            };
            int I0, J0, I1, J1;
            jobIJ(w, I0, J0);
            jobIJ(8 + (w & 1), I1, J1);
            const bool two = w < 2;
            f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = a0, x = a0, o = a0;
#pragma unroll
            for (int kk = 0; kk < KD; ++kk) {
                const bf16x8 sop = frag_rows(sm.S, PD, 16 * Jw, 32 * kk, lane);
                x = mfma32(frag_rows(sm.K, PD, 16 * Iw, 32 * kk, lane), sop, x);
                o = mfma32(frag_rows(sm.Q, PD, 16 * Iw, 32 * kk, lane), sop, o);
                a0 = mfma32(frag_rows(sm.K, PD, 16 * I0, 32 * kk, lane),
                            frag_rows(Bop, PD, 16 * J0, 32 * kk, lane), a0);
                if (two)
                    a1 = mfma32(frag_rows(sm.K, PD, 16 * I1, 32 * kk, lane),
                                frag_rows(Bop, PD, 16 * J1, 32 * kk, lane), a1);
            }
            // L^T[s][r] = beta_r * A[r][s] (s < r), zero elsewhere
            auto putL = [&](int I, int J, f32x4 acc) {
                const int s = 16 * J + l15;
                const int r0 = 16 * I + 4 * l4;
                const f32x4 br = *reinterpret_cast<const f32x4 *>(&sm.beta[r0]);
                f32x4 val;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = r0 + e;
                    float dv = 1.f;
                    if (!CH) dv = ex(fminf(sm.gb[r] - sm.gb[s], 0.f));
                    val[e] = s < r ? acc[e] * dv * br[e] : 0.f;
                }
                *reinterpret_cast<f32x4 *>(&sm.LT[s * PL + r0]) = val;
            };
            putL(I0, J0, a0);
            if (two) putL(I1, J1, a1);
            // X = V - Kt S0^T  (GDN: Kt S0^T = diag(e^b) k S0^T)
            const int iv = 16 * Jw + l15;
            const int r0 = 16 * Iw + 4 * l4;
            f32x4 xv;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float gr = CH ? 1.f : ex(sm.gb[r0 + e]);
                xv[e] = (float)sm.V[(r0 + e) * PV + iv] - gr * x[e];
                o[e] *= gr;
            }
            *reinterpret_cast<bf16x4 *>(&sm.XT[iv * PC + r0]) = cvt4(xv);
            accO = o;
        }
        __syncthreads();

        // ================= 3: T (wave 0) || P (waves 1-7) =================
        if (w == 0) {
            // diagonal blocks: lane = (block b, column cc); right-looking
            // forward substitution of (I + L_bb) y = e_cc in fp32
            const int b = l4;
            const int cc = l15;
            float y[16], acc[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                y[r] = r == cc ? 1.f : (r > cc ? -acc[r] : 0.f);
                // column r of L_bb = row r of L^T_bb
                const float *lt = &sm.LT[(16 * b + r) * PL + 16 * b];
#pragma unroll
                for (int q4 = (r + 1) / 4; q4 < 4; ++q4) {
                    const f32x4 col = *reinterpret_cast<const f32x4 *>(lt + 4 * q4);
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (4 * q4 + e > r) acc[4 * q4 + e] += col[e] * y[r];
                }
            }
            const float bcc = sm.beta[16 * b + cc];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                sm.Y[(b * 16 + r) * PY + cc] = y[r];
                sm.Tm[(16 * b + r) * PC + 16 * b + cc] = (bf16)(y[r] * bcc);
            }
            __threadfence_block();
            // off-diagonal blocks, Y_ij = -Y_ii sum_{k=j}^{i-1} L_ik Y_kj, on
            // 16x16x16 MFMAs.  A operand: row l15, cols 4*l4..+3; B operand:
            // rows 4*l4..+3, col l15 (== the accumulator layout).
            auto opL = [&](int bi, int bk) -> bf16x4 {   // L_ik rows: L^T columns
                const float *p = &sm.LT[(16 * bk + 4 * l4) * PL + 16 * bi + l15];
                return bf16x4{(bf16)p[0], (bf16)p[PL], (bf16)p[2 * PL], (bf16)p[3 * PL]};
            };
            auto opYA = [&](int bi) -> bf16x4 {
                return cvt4(*reinterpret_cast<const f32x4 *>(&sm.Y[(bi * 16 + l15) * PY + 4 * l4]));
            };
            auto opYB = [&](int bj) -> bf16x4 {
                const float *p = &sm.Y[(bj * 16 + 4 * l4) * PY + l15];
                return bf16x4{(bf16)p[0], (bf16)p[PY], (bf16)p[2 * PY], (bf16)p[3 * PY]};
            };
            const f32x4 z0 = {0.f, 0.f, 0.f, 0.f};
            const bf16x4 Y00 = opYB(0), Y11 = opYB(1), Y22 = opYB(2);
            const bf16x4 A11 = opYA(1), A22 = opYA(2), A33 = opYA(3);
            const bf16x4 L10 = opL(1, 0), L21 = opL(2, 1), L32 = opL(3, 2);
            const bf16x4 L20 = opL(2, 0), L31 = opL(3, 1), L30 = opL(3, 0);
            const f32x4 Y10 = -mfma16(A11, cvt4(mfma16(L10, Y00, z0)), z0);
            const f32x4 Y21 = -mfma16(A22, cvt4(mfma16(L21, Y11, z0)), z0);
            const f32x4 Y32 = -mfma16(A33, cvt4(mfma16(L32, Y22, z0)), z0);
            const f32x4 Y20 = -mfma16(A22, cvt4(mfma16(L21, cvt4(Y10), mfma16(L20, Y00, z0))), z0);
            const f32x4 Y31 = -mfma16(A33, cvt4(mfma16(L32, cvt4(Y21), mfma16(L31, Y11, z0))), z0);
            const f32x4 Y30 = -mfma16(
                A33, cvt4(mfma16(L32, cvt4(Y20), mfma16(L31, cvt4(Y10), mfma16(L30, Y00, z0)))), z0);
            auto put = [&](int bi, int bj, f32x4 yv) {
                const int s = 16 * bj + l15;
                const float bs = sm.beta[s];
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    sm.Tm[(16 * bi + 4 * l4 + e) * PC + s] = (bf16)(yv[e] * bs);
            };
            put(1, 0, Y10);
            put(2, 1, Y21);
            put(3, 2, Y32);
            put(2, 0, Y20);
            put(3, 1, Y31);
            put(3, 0, Y30);
        } else {
            // P jobs 0..9 over waves 1..7: job w-1, and job w+6 for w <= 3
            auto jobIJ = [](int tri, int &I, int &J) {
                I = tri < 1 ? 0 : tri < 3 ? 1 : tri < 6 ? 2 : 3;
                J = tri - I * (I + 1) / 2;
            };
            int I0, J0, I1, J1;
            jobIJ(w - 1, I0, J0);
            jobIJ(w <= 3 ? w + 6 : 9, I1, J1);
            const bool two = w <= 3;
            f32x4 p0 = {0.f, 0.f, 0.f, 0.f}, p1 = p0;
#pragma unroll
            for (int kk = 0; kk < KD; ++kk) {
                p0 = mfma32(frag_rows(sm.Q, PD, 16 * I0, 32 * kk, lane),
                            frag_rows(Bop, PD, 16 * J0, 32 * kk, lane), p0);
                if (two)
                    p1 = mfma32(frag_rows(sm.Q, PD, 16 * I1, 32 * kk, lane),
                                frag_rows(Bop, PD, 16 * J1, 32 * kk, lane), p1);
            }
            auto putP = [&](int I, int J, f32x4 acc) {
                const int s = 16 * J + l15;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 16 * I + 4 * l4 + e;
                    float dv = 1.f;
                    if (!CH) dv = ex(fminf(sm.gb[r] - sm.gb[s], 0.f));
                    sm.P[r * PC + s] = (bf16)(s <= r ? acc[e] * dv : 0.f);
                }
            };
            putP(I0, J0, p0);
            if (two) putP(I1, J1, p1);
        }
        __syncthreads();

        // ================= 4: U = T X =====================================
        {
            f32x4 u = {0.f, 0.f, 0.f, 0.f};
            u = mfma32(frag_rows(sm.Tm, PC, 16 * Iw, 0, lane),
                       frag_rows(sm.XT, PC, 16 * Jw, 0, lane), u);
            if (Iw >= 2)   // T is lower triangular: rows < 32 need s < 32 only
                u = mfma32(frag_rows(sm.Tm, PC, 16 * Iw, 32, lane),
                           frag_rows(sm.XT, PC, 16 * Jw, 32, lane), u);
            *reinterpret_cast<bf16x4 *>(&sm.UT[(16 * Jw + l15) * PC + 16 * Iw + 4 * l4]) = cvt4(u);
        }
        __syncthreads();

        // ================= 5: outputs and the next state ==================
        {
            f32x4 o = accO;
            o = mfma32(frag_rows(sm.P, PC, 16 * Iw, 0, lane),
                       frag_rows(sm.UT, PC, 16 * Jw, 0, lane), o);
            if (Iw >= 2)
                o = mfma32(frag_rows(sm.P, PC, 16 * Iw, 32, lane),
                           frag_rows(sm.UT, PC, 16 * Jw, 32, lane), o);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * Iw + 4 * l4 + e;
                if (r < Cc) og[(size_t)(tc + r) * tokstride + 16 * Jw + l15] = (bf16)(a.scale * o[e]);
            }
        }
#pragma unroll
        for (int sb = 0; sb < SB; ++sb) {
            const int Jk = jk_of(sb);
            const int Jv = jv_of(sb);
            const int j = 16 * Jk + 4 * l4;
            f32x4 gm;
            if (CH) gm = *reinterpret_cast<const f32x4 *>(&sm.gam[j]);
            else    gm = f32x4{sm.gam[0], sm.gam[0], sm.gam[0], sm.gam[0]};
            f32x4 s = St[sb] * gm;
#pragma unroll
            for (int kk = 0; kk < C / 32; ++kk)
                s = mfma32(frag_cols(sm.Kh, PD, 32 * kk, 16 * Jk, lane),
                           frag_rows(sm.UT, PC, 16 * Jv, 32 * kk, lane), s);
            St[sb] = s;
            *reinterpret_cast<bf16x4 *>(&sm.S[(16 * Jv + l15) * PD + j]) = cvt4(s);
        }
    }

    if (a.ht) {
#pragma unroll
        for (int sb = 0; sb < SB; ++sb) {
            const int j = 16 * jk_of(sb) + 4 * l4;
            const int iv = 16 * jv_of(sb) + l15;
            *reinterpret_cast<f32x4 *>(a.ht + sslot + (size_t)(i0 + iv) * D + j) = St[sb];
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
    dim3 grid((unsigned)blocks), block(NT);
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
