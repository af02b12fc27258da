// backward.hip -- gradients of the chunked gated delta rule on gfx950.
//
// Forward, per sequence and head ("Super Apriel: One Checkpoint, Many
// Speeds", gist.science summary 2a, for the two gate kinds):
//     S_t = S_{t-1} Diag(a_t)(I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
//     o_t = scale * S_t q_t,   a_t = e^{g_t}.
// For upstream gradients dO (of o) and dS_T (of the final state) the
// backward returns dq, dk, dv, dg, dbeta and dS_0 in three stages, for a
// fixed-length or a packed batch alike (per-chunk data is indexed by global
// chunk, the chunks of all sequences numbered one after the other):
//
// 1. the chunked forward (chunked.hip / chunked_chain.hip) with its
//    optional output of the state entering every chunk of 64 tokens.
// 2. chunk_grad_kernel<.., PREP>: per (chunk, head), the chunk-local
//    matrices of the state gradient's recurrence (below) into a record;
//    adjoint_chain_kernel: that recurrence chunk by chunk in reverse,
//        dS_{c-1} = dS_c Diag(e^{b_C}) + scale dO^T Qt - dU^T W,
//        dU = Kb (dS_c Diag(e^{b_C}))^T + scale P^T dO,  W = T Kt,
//    from dS_{last} = dS_T; it stores every chunk's dS_C and dS_0.
// 3. chunk_grad_kernel: per (chunk, head), from the entering state S0 and
//    dS_C, every input gradient of the chunk by differentiating the chunked
//    form (see chunked.hip) -- with b the in-chunk cumulative log gate,
//    E = e^b, Qt = q.E, Kt = k.E, Kb = k/E, Kh = Kb e^{b_C}:
//        A = strict_lower(Kt Kb^T), P = lower(Qt Kb^T),
//        N = (I + diag(beta) A)^{-1}, T = N diag(beta),
//        X = V - Kt S0^T, U = T X,
//        O = scale (Qt S0^T + P U),  S_C = S0 Diag(e^{b_C}) + U^T Kh.
//    With dSg = dS_C Diag(e^{b_C}):
//        dU  = Kb dSg^T + scale P^T dO          dKh.Kh / Kb = U dSg
//        dP  = scale lower(dO U^T)              dQt = scale dO S0 + dP Kb
//        dT  = lower(dU X^T)                    dX  = T^T dU = dV
//        dN  = dT diag(beta)                    dbeta_s += sum_r dT_rs N_rs
//        dM  = -N^T dN N^T                      dA  = strict_lower(diag(beta) dM)
//        dbeta_r += sum_s dM_rs A_rs
//        dKt = -dX S0 + dA Kb                   dKb = dP^T Qt + dA^T Kt + U dSg
//        dq = dQt.E,  dk = dKt.E + dKb/E,  db_r = dQt.Qt + dKt.Kt - dKb.Kb
//        db_C = sum_r (U dSg).Kb + sum_i dSg_i.S0_i
//        dg_s = sum_{r >= s} db_r + db_C     (summed over channels for GDN)
//    The Kh part h_r = (U dSg).Kb enters db_r with a minus sign and db_C
//    with a plus sign; summed, it adds sum_{r < s} h_r to dg_s, which is how
//    it is computed (the two large terms would otherwise cancel in bf16).
//    The products run on 16x16x32 bf16 MFMAs with fp32 accumulation (the
//    fp32 states S0 and dS_C as hi + lo bf16 pairs); the triangular inverse
//    by substitution in fp32.  The diagonals of T and dP, rounded once to
//    bf16 as operands, get their rounding error added back in fp32 (in a
//    short chunk they carry most of the weight, and one rounding of them is
//    a correlated error in everything downstream).
#include "gdr_internal.h"
#include "device_util.h"

namespace gdr {
namespace {

constexpr int C = 64;

// ===========================================================================
// chunk_grad_kernel
// ===========================================================================
constexpr int PC = C + 8;     // row length of the C x C bf16 matrices in LDS

template <int D> struct GradSmem {
    static constexpr int PD = D + 8;
    alignas(16) bf16 Qt[C * PD];      // q e^b            [r][j]
    alignas(16) bf16 Kt[C * PD];      // k e^b
    alignas(16) bf16 Kb[C * PD];      // k e^-b
    static constexpr int PQ = 32 + 8;  // row length of a C x 32 slice
    // one region, used in turn by the steps
    union alignas(16) {
        char stage[C * D * 8];        // step 1: q, k (bf16) and g (fp32) of the chunk
        struct {
            float Nf[C * C];          // L, then N = (I + L)^{-1}  [r][s]
            float L[9 * 256];         // blocks of L below the diagonal, products
        } inv;                        // steps 2, 3
        struct {                      // steps 4-13, 32 value columns i at a time
            bf16 S0h[32 * PD], S0l[32 * PD];   // S0 rows i of the slice, hi + lo
            bf16 dSh[32 * PD], dSl[32 * PD];   // dSg likewise
            bf16 X[C * PQ], U[C * PQ], dU[C * PQ], dO[C * PQ], dX[C * PQ];   // [r][i]
        } sl;
        float db[C * D];              // step 16
    } R;
    alignas(16) bf16 Tb[C * PC];      // T, later Y = dN N^T
    alignas(16) bf16 Pb[C * PC];      // P, later dN
    alignas(16) bf16 dPb[C * PC];     // dP, later dA
    alignas(16) bf16 Nb[C * PC];      // N
    alignas(16) float beta[C];
    alignas(16) float eC[D];          // e^{b_C} per channel (scalar gate: all equal)
    alignas(16) float dbC[D];         // gradient of b_C per channel
    alignas(16) float dbeta[C];
    alignas(16) float dbrow[C];       // scalar gate: db per row
    alignas(16) float hrow[C];        // scalar gate: Kh part of db per row
    alignas(16) float tcor[C];        // T_rr - bf16(T_rr): the diagonal of T is beta
    alignas(16) float pcor[C];        // dP_rr - bf16(dP_rr)
    alignas(16) float bs[C];          // scalar gate: b per row
};

// MFMA fragments from global memory: fp32 row-major [rows][ld] (rows of the
// fragment along the matrix rows) and its column form, bf16 likewise; rows
// at or past `valid` read as zeros.  The fp32 ones (the states and their
// gradients) come as a pair hi + lo of bf16 values, hi = bf16(x) and
// lo = bf16(x - hi), so that two MFMAs carry about 16 bits of x: the
// gate gradient sums terms that cancel to a fraction of their size.
struct Frag2 {
    bf16x8 hi, lo;
};
__device__ inline Frag2 split8(const float (&v)[8]) {
    Frag2 f;
    f.hi = cvt8(v);
    float r[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) r[u] = v[u] - (float)f.hi[u];
    f.lo = cvt8(r);
    return f;
}
__device__ inline Frag2 g_rows_f32(const float *base, size_t ld, int r0, int k0, int lane,
                                   const float *cs) {
    const float *p = base + (size_t)(r0 + (lane & 15)) * ld + k0 + 8 * (lane >> 4);
    const f32x4 x0 = *reinterpret_cast<const f32x4 *>(p);
    const f32x4 x1 = *reinterpret_cast<const f32x4 *>(p + 4);
    float v[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
    if (cs) {
        const float *c = cs + k0 + 8 * (lane >> 4);
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] *= c[u];
    }
    return split8(v);
}
__device__ inline Frag2 g_cols_f32(const float *base, size_t ld, int k0, int n0, int lane,
                                   float cscale) {
    const float *p = base + (size_t)(k0 + 8 * (lane >> 4)) * ld + n0 + (lane & 15);
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = p[(size_t)u * ld] * cscale;
    return split8(v);
}
// A x (hi + lo), A as the first operand; (hi + lo) x B
__device__ inline f32x4 mfma_ab2(bf16x8 a, const Frag2 &b, f32x4 c) {
    return mfma32(a, b.lo, mfma32(a, b.hi, c));
}
__device__ inline bf16x8 g_rows_bf(const bf16 *base, size_t ld, int r0, int k0, int lane, int valid) {
    const int r = r0 + (lane & 15);
    if (r >= valid) return bf16x8{};
    return *reinterpret_cast<const bf16x8 *>(base + (size_t)r * ld + k0 + 8 * (lane >> 4));
}
__device__ inline bf16x8 g_cols_bf(const bf16 *base, size_t ld, int k0, int n0, int lane, int valid) {
    const int kb = k0 + 8 * (lane >> 4);
    const bf16 *p = base + n0 + (lane & 15);
    bf16x8 v;
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = kb + u < valid ? p[(size_t)(kb + u) * ld] : (bf16)0.f;
    return v;
}

// sum of x over the four lanes (l & 15) + 16 m, m = 0..3
__device__ inline float sum_quads(float x) { return swap_sum32(swap_sum16(x)); }

// Per-chunk record of the adjoint chain: the chunk-local matrices that the
// state gradient's recurrence needs, in bf16, and e^{b_C} in fp32.
template <int D> struct ChainRec {
    static constexpr size_t QT = 0;                          // Qt [C][D]
    static constexpr size_t KB = QT + (size_t)C * D * 2;     // Kb [C][D]
    static constexpr size_t W = KB + (size_t)C * D * 2;      // W = T Kt [C][D]
    static constexpr size_t P = W + (size_t)C * D * 2;       // P [C][C]
    static constexpr size_t EC = P + (size_t)C * C * 2;      // e^{b_C} [D] fp32
    static constexpr size_t BYTES = EC + (size_t)D * 4;
};

// Channel gate: b = running sums down the rows of the chunk's g [C][D]
// (global, token stride gstr, rows at or past Cc as zeros), into gs [C][D]
// in LDS.  All NT threads load with 16-byte loads; then NT / D parts of
// the rows per channel are summed by one thread each and offset by the
// parts above (tot: NT floats of LDS).  Ends with a barrier.
template <int D, int NT>
__device__ inline void gate_load(f32x4 (&gv)[C * D / 4 / NT], const float *gg, size_t gstr, int Cc,
                                 int tid) {
#pragma unroll
    for (int it = 0; it < C * D / 4 / NT; ++it) {
        const int p = it * NT + tid, r = p / (D / 4), j = 4 * (p % (D / 4));
        gv[it] = r < Cc ? *reinterpret_cast<const f32x4 *>(gg + (size_t)r * gstr + j) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int u = 0; u < 4; ++u) gv[it][u] = __builtin_fmaxf(gv[it][u], kGateFloor);   // as the forward
    }
}
template <int D, int NT>
__device__ inline void gate_sums_from(float *gs, float *tot, const f32x4 (&gv)[C * D / 4 / NT], int tid) {
#pragma unroll
    for (int it = 0; it < C * D / 4 / NT; ++it) {
        const int p = it * NT + tid, r = p / (D / 4), j = 4 * (p % (D / 4));
        *reinterpret_cast<f32x4 *>(gs + r * D + j) = gv[it];
    }
    __syncthreads();
    constexpr int NH = NT / D, RH = C / NH;
    const int j = tid % D, part = tid / D;
    float rs[RH], run = 0.f;
#pragma unroll
    for (int u = 0; u < RH; ++u) {
        run += gs[(part * RH + u) * D + j];
        rs[u] = run;
    }
    tot[part * D + j] = run;
    __syncthreads();
    float off = 0.f;
    for (int q = 0; q < part; ++q) off += tot[q * D + j];
#pragma unroll
    for (int u = 0; u < RH; ++u) gs[(part * RH + u) * D + j] = rs[u] + off;
    __syncthreads();
}
template <int D, int NT>
__device__ inline void gate_running_sums(float *gs, float *tot, const float *gg, size_t gstr, int Cc, int tid) {
    f32x4 gv[C * D / 4 / NT];
    gate_load<D, NT>(gv, gg, gstr, Cc, tid);
    gate_sums_from<D, NT>(gs, tot, gv, tid);
}

// The chunks of all sequences are numbered one after the other: sequence n's
// chunk c is global chunk base_n + c (fixed length: n nc + c).  Per global
// chunk: its sequence, its index in the sequence, the sequence's first token
// and length; false past the last chunk (packed batches: the grid is sized
// for an upper bound).
struct ChunkLoc {
    int n, c;
    long long seq0, len;
};
__device__ inline bool locate_chunk(const BwdArgs &a, long long gc, ChunkLoc &L) {
    if (a.cu_seqlens) {
        if (gc >= a.chunk_base[a.B]) return false;
        int lo = 0, hi = a.B;                  // chunk_base[lo] <= gc < chunk_base[hi]
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (a.chunk_base[mid] <= gc) lo = mid;
            else hi = mid;
        }
        L.n = lo;
        L.c = (int)(gc - a.chunk_base[lo]);
        L.seq0 = a.cu_seqlens[lo];
        L.len = a.cu_seqlens[lo + 1] - L.seq0;
    } else {
        L.n = (int)(gc / a.nc);
        L.c = (int)(gc - (long long)L.n * a.nc);
        L.seq0 = (long long)L.n * a.T;
        L.len = a.T;
    }
    return true;
}

// PREP: stop after T and write the chunk's ChainRec (no S0 or dS_C needed).
template <int D, bool CH, bool PREP>
__global__ __launch_bounds__(512) void chunk_grad_kernel(BwdArgs a) {
    using Sm = GradSmem<D>;
    constexpr int PD = Sm::PD;
    constexpr int KD = D / 32;         // 32-wide k steps over D
    constexpr int NB = D / 16;         // 16-wide column blocks of a C x D matrix
    constexpr int NT = 512;            // eight waves: two per row block I, each
    constexpr int NBH = NB / 2;        // with half of the column blocks (or of J)
    __shared__ Sm sm;

    const int h = blockIdx.x % a.H;
    const long long gc = blockIdx.x / a.H;    // global chunk
    ChunkLoc loc;
    if (!locate_chunk(a, gc, loc)) return;
    const int t0 = loc.c * C;
    const int Cc = loc.len - t0 < C ? (int)(loc.len - t0) : C;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int half = w >> 2, cb0 = half * NBH;
    const int l15 = lane & 15, q4 = lane >> 4;
    const size_t rowD = (size_t)a.H * D;                      // token stride of q, k, v, o
    const size_t tok0 = (size_t)(loc.seq0 + t0);              // first token row
    const bf16 *qg = static_cast<const bf16 *>(a.q) + (tok0 * a.H + h) * D;
    const bf16 *kg = static_cast<const bf16 *>(a.k) + (tok0 * a.H + h) * D;
    const bf16 *vg = static_cast<const bf16 *>(a.v) + (tok0 * a.H + h) * D;
    const bf16 *dog = static_cast<const bf16 *>(a.dout) + (tok0 * a.H + h) * D;
    const size_t gstr = CH ? rowD : (size_t)a.H;              // token stride of g
    const float *gg = a.g + (CH ? (tok0 * a.H + h) * D : tok0 * a.H + h);
    const float *bg = a.beta + tok0 * a.H + h;
    const size_t sbh = (size_t)gc * a.H + h;                  // [chunk][head] records
    const float *S0 = a.states + sbh * D * D;                  // [i][j]
    const float *dSC = a.dstates + sbh * D * D;                // [i][j]
    float *const Nf = sm.R.inv.Nf;

    // ---- 1. gate sums, gated operands, beta; zero the accumulators
    if (tid < C) {
        sm.beta[tid] = tid < Cc ? bg[(size_t)tid * a.H] : 0.f;
        sm.dbeta[tid] = 0.f;
        sm.dbrow[tid] = 0.f;
        sm.hrow[tid] = 0.f;
    }
    if (!CH && w == 0) {
        const float gv = lane < Cc ? __builtin_fmaxf(gg[(size_t)lane * gstr], kGateFloor) : 0.f;
        sm.bs[lane] = wave_prefix_sum(gv);
    }
    if (tid < D) sm.dbC[tid] = 0.f;
    // q and k of the chunk in registers (16-byte loads from all threads, all
    // in flight together), the channel gate g in LDS, rows past the end as
    // zeros
    constexpr int NQ = C * D / 8 / NT;         // 16-byte pieces of q per thread
    float *gst = reinterpret_cast<float *>(sm.R.stage);        // g, then b  [r][j]
    float *gtot = gst + C * D;                                 // part sums of g
    static_assert(sizeof(sm.R) >= sizeof(float) * (C * D + NT), "gate staging");
    bf16x8 qv[NQ], kv[NQ];
#pragma unroll
    for (int it = 0; it < NQ; ++it) {
        const int p = it * NT + tid, r = p / (D / 8), j = 8 * (p % (D / 8));
        qv[it] = kv[it] = bf16x8{};
        if (r < Cc) {
            qv[it] = *reinterpret_cast<const bf16x8 *>(qg + (size_t)r * rowD + j);
            kv[it] = *reinterpret_cast<const bf16x8 *>(kg + (size_t)r * rowD + j);
        }
    }
    if constexpr (CH) gate_running_sums<D, NT>(gst, gtot, gg, gstr, Cc, tid);
    else __syncthreads();
    // gated operands Qt = q e^b, Kt = k e^b, Kb = k e^-b
#pragma unroll
    for (int it = 0; it < NQ; ++it) {
        const int p = it * NT + tid, r = p / (D / 8), j = 8 * (p % (D / 8));
        float e[8];
        if constexpr (CH) {
            const f32x4 b0 = *reinterpret_cast<const f32x4 *>(gst + r * D + j);
            const f32x4 b1 = *reinterpret_cast<const f32x4 *>(gst + r * D + j + 4);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                e[u] = ex(b0[u]);
                e[u + 4] = ex(b1[u]);
            }
        } else {
            const float er = ex(sm.bs[r]);
#pragma unroll
            for (int u = 0; u < 8; ++u) e[u] = er;
        }
        bf16x8 qt, kt, kb;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const float qf = (float)qv[it][u], kf = (float)kv[it][u];
            qt[u] = (bf16)(qf * e[u]);
            kt[u] = (bf16)(kf * e[u]);
            kb[u] = (bf16)(kf * __builtin_amdgcn_rcpf(e[u]));
        }
        *reinterpret_cast<bf16x8 *>(&sm.Qt[r * PD + j]) = qt;
        *reinterpret_cast<bf16x8 *>(&sm.Kt[r * PD + j]) = kt;
        *reinterpret_cast<bf16x8 *>(&sm.Kb[r * PD + j]) = kb;
        if (r == C - 1) {
#pragma unroll
            for (int u = 0; u < 8; ++u) sm.eC[j + u] = e[u];
        }
    }
    __syncthreads();

    const int I = w & 3;                       // this wave's 16-row block
    auto zero4 = []() { return f32x4{0.f, 0.f, 0.f, 0.f}; };
    // r, s of accumulator element e of block (I, J)
    auto rowof = [&](int e) { return 16 * I + 4 * q4 + e; };

    // ---- 2. A = strict_lower(Kt Kb^T), P = lower(Qt Kb^T); L = diag(beta) A
#pragma unroll
    for (int Ji = 0; Ji < 2; ++Ji) {
        const int J = 2 * half + Ji;
        f32x4 av = zero4(), pv = zero4();
        if (J <= I) {
#pragma unroll
            for (int kk = 0; kk < KD; ++kk) {
                const bf16x8 kb = frag_rows(sm.Kb, PD, 16 * J, 32 * kk, lane);
                av = mfma32(frag_rows(sm.Kt, PD, 16 * I, 32 * kk, lane), kb, av);
                pv = mfma32(frag_rows(sm.Qt, PD, 16 * I, 32 * kk, lane), kb, pv);
            }
        }
        const int s = 16 * J + l15;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = rowof(e);
            if (!(s < r)) av[e] = 0.f;
            if (!(s <= r)) pv[e] = 0.f;
            const float lv = sm.beta[r] * av[e];
            Nf[r * C + s] = lv;
            if (J < I) sm.R.inv.L[(I * (I - 1) / 2 + J) * 256 + (4 * q4 + e) * 16 + l15] = lv;
            sm.Pb[r * PC + s] = (bf16)pv[e];
        }
    }
    __syncthreads();

    // ---- 3. N = (I + L)^{-1}, in fp32.  The 16x16 blocks of L below the
    //         diagonal are saved; the four
    //         diagonal blocks are inverted by substitution, lane 16 b + c of
    //         wave 0 taking column c of block b; then the blocks below the
    //         diagonal, N_ij = -N_ii sum_{k=j}^{i-1} L_ik N_kj, one block
    //         diagonal i - j = d at a time
    {
        const float *Ls = sm.R.inv.L;                  // [ltri(i, k)][16][16], from step 2
        float *Tm = sm.R.inv.L + 6 * 256;              // [3][16][16]
        if (w == 0) {
            const int base = 16 * (lane >> 4), c = lane & 15;
            float n[16];
            // row r of the block as four 16-byte reads (the same address
            // across the block's lanes), the next row's in flight
            auto lrow = [&](int r, f32x4 (&L)[4]) {
#pragma unroll
                for (int v = 0; v < 4; ++v) L[v] = *reinterpret_cast<const f32x4 *>(&Nf[(base + r) * C + base + 4 * v]);
            };
            f32x4 Lc[4], Ln[4];
            lrow(0, Lc);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                if (r + 1 < 16) lrow(r + 1, Ln);
                float acc = r == c ? 1.f : 0.f;
#pragma unroll
                for (int m = 0; m < r; ++m) acc -= Lc[m >> 2][m & 3] * n[m];
                n[r] = acc;
#pragma unroll
                for (int v = 0; v < 4; ++v) Lc[v] = Ln[v];
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) Nf[(base + r) * C + base + c] = n[r];
        }
        __syncthreads();
        // wave w takes block (w + d, w), on fp32 MFMAs (16x16x4: lane l holds
        // A[l & 15][l >> 4], B[l >> 4][l & 15]); the product L N through a
        // wave-private block of LDS into the layout of an operand
        for (int d = 1; d < 4; ++d) {
            const int jb = w, ib = w + d;
            if (ib < 4) {
                float *Tw = Tm + w * 256;
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                for (int kb = jb; kb < ib; ++kb) {
                    const float *L = Ls + (ib * (ib - 1) / 2 + kb) * 256;
#pragma unroll
                    for (int kk = 0; kk < 4; ++kk)
                        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(L[l15 * 16 + 4 * kk + q4],
                                                                   Nf[(16 * kb + 4 * kk + q4) * C + 16 * jb + l15], acc, 0, 0, 0);
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) Tw[(4 * q4 + e) * 16 + l15] = acc[e];
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
                f32x4 n = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < 4; ++kk)
                    n = __builtin_amdgcn_mfma_f32_16x16x4f32(Nf[(16 * ib + l15) * C + 16 * ib + 4 * kk + q4],
                                                             Tw[(4 * kk + q4) * 16 + l15], n, 0, 0, 0);
#pragma unroll
                for (int e = 0; e < 4; ++e) Nf[(16 * ib + 4 * q4 + e) * C + 16 * jb + l15] = -n[e];
            }
            __syncthreads();
        }
    }
    // N and T = N diag(beta) to bf16, four consecutive entries per thread
    // and read (a wave reads 1 KiB of consecutive LDS per instruction)
#pragma unroll
    for (int it = 0; it < C * C / 4 / NT; ++it) {
        const int p = it * NT + tid, r = p / (C / 4), s0 = 4 * (p % (C / 4));
        const f32x4 nv = *reinterpret_cast<const f32x4 *>(&Nf[r * C + s0]);
        const f32x4 bv = *reinterpret_cast<const f32x4 *>(&sm.beta[s0]);
        bf16x4 nb, tb;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const float tv = nv[u] * bv[u];
            nb[u] = (bf16)nv[u];
            tb[u] = (bf16)tv;
            if (s0 + u == r) sm.tcor[r] = tv - (float)tb[u];
        }
        *reinterpret_cast<bf16x4 *>(&sm.Nb[r * PC + s0]) = nb;
        *reinterpret_cast<bf16x4 *>(&sm.Tb[r * PC + s0]) = tb;
    }
    __syncthreads();

    if constexpr (PREP) {
        // W = T Kt (the diagonal of T compensated), then the record
        using R = ChainRec<D>;
        char *rec = static_cast<char *>(a.recs) + sbh * R::BYTES;
        bf16 *Wg = reinterpret_cast<bf16 *>(rec + R::W);
#pragma unroll
        for (int cbi = 0; cbi < NBH; ++cbi) {
            const int cb = cb0 + cbi;
            f32x4 x = zero4();
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
                x = mfma32(frag_rows(sm.Tb, PC, 16 * I, 32 * kk, lane), frag_cols(sm.Kt, PD, 32 * kk, 16 * cb, lane), x);
            const int j = 16 * cb + l15;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = rowof(e);
                Wg[r * D + j] = (bf16)(x[e] + sm.tcor[r] * (float)sm.Kt[r * PD + j]);
            }
        }
        bf16 *Qg = reinterpret_cast<bf16 *>(rec + R::QT);
        bf16 *Kg = reinterpret_cast<bf16 *>(rec + R::KB);
        for (int p = tid; p < C * D / 8; p += NT) {
            const int r = p / (D / 8), j = 8 * (p % (D / 8));
            *reinterpret_cast<bf16x8 *>(Qg + r * D + j) = *reinterpret_cast<const bf16x8 *>(&sm.Qt[r * PD + j]);
            *reinterpret_cast<bf16x8 *>(Kg + r * D + j) = *reinterpret_cast<const bf16x8 *>(&sm.Kb[r * PD + j]);
        }
        bf16 *Pg = reinterpret_cast<bf16 *>(rec + R::P);
        for (int p = tid; p < C * C / 8; p += NT) {
            const int r = p / (C / 8), sc = 8 * (p % (C / 8));
            *reinterpret_cast<bf16x8 *>(Pg + r * C + sc) = *reinterpret_cast<const bf16x8 *>(&sm.Pb[r * PC + sc]);
        }
        if (tid < D) reinterpret_cast<float *>(rec + R::EC)[tid] = sm.eC[tid];
        return;
    }

    // ---- 4-13. The products with S0 and dSg, 32 value columns i at a
    //         time.  Each slice -- rows i of S0 and dSg (as hi + lo bf16,
    //         dSg = dS_C with the column scale e^{b_C}) and columns i of V
    //         and dO -- is staged in LDS once, the next slice's loads in
    //         flight meanwhile.  X, U, dU and dX = dV are column-local
    //         (U = T X, dX = T^T dU), so only their slice is kept; the
    //         products over i (dT, dP, dQt, dKt, dKbh) accumulate in
    //         registers.  db_C's S0 part, sum_i dSg_i.S0_i, is summed from
    //         the fp32 loads.
    float Nreg[2][4];                          // N of this wave's blocks, in fp32
#pragma unroll
    for (int Ji = 0; Ji < 2; ++Ji)
#pragma unroll
        for (int e = 0; e < 4; ++e) Nreg[Ji][e] = Nf[rowof(e) * C + 16 * (2 * half + Ji) + l15];
    __syncthreads();                           // Nf no longer read

    auto &sl = sm.R.sl;
    constexpr int PQ = Sm::PQ;
    constexpr int NS4 = 32 * D / 4 / NT;       // 16-byte pieces of a state slice per thread
    f32x4 ps[NS4], pd[NS4];
    bf16x8 pv, po;
    float dbc[4] = {0.f, 0.f, 0.f, 0.f};       // columns jc .. jc + 3 of db_C
    const int jc = 4 * (tid % (D / 4));
    const bool vown = tid < 256;               // threads staging the V and dO slices
    const int vr = (tid & 255) >> 2, vc = 8 * (tid & 3);   // their row, column in the slice
    auto fetch = [&](int sc) {
#pragma unroll
        for (int it = 0; it < NS4; ++it) {
            const int ii = (it * NT + tid) / (D / 4);
            const size_t o = (size_t)(32 * sc + ii) * D + jc;
            ps[it] = *reinterpret_cast<const f32x4 *>(S0 + o);
            pd[it] = *reinterpret_cast<const f32x4 *>(dSC + o);
        }
        pv = po = bf16x8{};
        if (vown && vr < Cc) {
            pv = *reinterpret_cast<const bf16x8 *>(vg + (size_t)vr * rowD + 32 * sc + vc);
            po = *reinterpret_cast<const bf16x8 *>(dog + (size_t)vr * rowD + 32 * sc + vc);
        }
    };
    auto put = [&]() {
        const f32x4 ec = *reinterpret_cast<const f32x4 *>(&sm.eC[jc]);
#pragma unroll
        for (int it = 0; it < NS4; ++it) {
            const int ii = (it * NT + tid) / (D / 4);
            bf16x4 sh, sl4, dh, dl;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const float sv = ps[it][u], dv = pd[it][u] * ec[u];
                dbc[u] += sv * dv;
                sh[u] = (bf16)sv;
                sl4[u] = (bf16)(sv - (float)sh[u]);
                dh[u] = (bf16)dv;
                dl[u] = (bf16)(dv - (float)dh[u]);
            }
            *reinterpret_cast<bf16x4 *>(&sl.S0h[ii * PD + jc]) = sh;
            *reinterpret_cast<bf16x4 *>(&sl.S0l[ii * PD + jc]) = sl4;
            *reinterpret_cast<bf16x4 *>(&sl.dSh[ii * PD + jc]) = dh;
            *reinterpret_cast<bf16x4 *>(&sl.dSl[ii * PD + jc]) = dl;
        }
        if (vown) {
            *reinterpret_cast<bf16x8 *>(&sl.X[vr * PQ + vc]) = pv;
            *reinterpret_cast<bf16x8 *>(&sl.dO[vr * PQ + vc]) = po;
        }
    };

    // column blocks cb0 + cbi and row blocks J = 2 half + Ji of this wave
    f32x4 dQt[NBH], dKt[NBH], dKb[NBH], dKbh[NBH], dPa[2], dTa[2];
#pragma unroll
    for (int cbi = 0; cbi < NBH; ++cbi) dQt[cbi] = dKt[cbi] = dKbh[cbi] = zero4();
#pragma unroll
    for (int Ji = 0; Ji < 2; ++Ji) dPa[Ji] = dTa[Ji] = zero4();
    fetch(0);
    for (int sc = 0; sc < D / 32; ++sc) {
        put();
        if (sc + 1 < D / 32) fetch(sc + 1);
        __syncthreads();
        // X = V - Kt S0^T and dU = Kb dSg^T + scale P^T dO on the slice
        {
            const int cl = half;
            f32x4 x = zero4(), du = zero4(), dp = zero4();
#pragma unroll
            for (int kk = 0; kk < KD; ++kk) {
                x = mfma_ab2(frag_rows(sm.Kt, PD, 16 * I, 32 * kk, lane),
                             Frag2{frag_rows(sl.S0h, PD, 16 * cl, 32 * kk, lane),
                                   frag_rows(sl.S0l, PD, 16 * cl, 32 * kk, lane)}, x);
                du = mfma_ab2(frag_rows(sm.Kb, PD, 16 * I, 32 * kk, lane),
                              Frag2{frag_rows(sl.dSh, PD, 16 * cl, 32 * kk, lane),
                                    frag_rows(sl.dSl, PD, 16 * cl, 32 * kk, lane)}, du);
            }
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
                dp = mfma32(frag_cols(sm.Pb, PC, 32 * kk, 16 * I, lane), frag_cols(sl.dO, PQ, 32 * kk, 16 * cl, lane), dp);
            const int il = 16 * cl + l15;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = rowof(e);
                sl.X[r * PQ + il] = (bf16)((float)sl.X[r * PQ + il] - x[e]);
                sl.dU[r * PQ + il] = (bf16)(du[e] + a.scale * dp[e]);
            }
        }
        __syncthreads();
        // U = T X, dX = T^T dU (= dV; the diagonal of T compensated), dT += dU X^T
        {
            const int cl = half;
            f32x4 u = zero4(), dx = zero4();
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                u = mfma32(frag_rows(sm.Tb, PC, 16 * I, 32 * kk, lane), frag_cols(sl.X, PQ, 32 * kk, 16 * cl, lane), u);
                dx = mfma32(frag_cols(sm.Tb, PC, 32 * kk, 16 * I, lane), frag_cols(sl.dU, PQ, 32 * kk, 16 * cl, lane), dx);
            }
            const int il = 16 * cl + l15, i = 32 * sc + il;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = rowof(e);
                sl.U[r * PQ + il] = (bf16)(u[e] + sm.tcor[r] * (float)sl.X[r * PQ + il]);
                const float dxv = dx[e] + sm.tcor[r] * (float)sl.dU[r * PQ + il];
                sl.dX[r * PQ + il] = (bf16)dxv;
                if (r < Cc) a.dv[((tok0 + r) * a.H + h) * D + i] = dxv;
            }
        }
        {
            const bf16x8 du = frag_rows(sl.dU, PQ, 16 * I, 0, lane);
#pragma unroll
            for (int Ji = 0; Ji < 2; ++Ji) {
                const int J = 2 * half + Ji;
                if (J <= I) dTa[Ji] = mfma32(du, frag_rows(sl.X, PQ, 16 * J, 0, lane), dTa[Ji]);
            }
        }
        __syncthreads();
        // dP += dO U^T;  over the slice's rows of S0 and dSg: dQt += dO S0,
        // dKt += dX S0 (negated below), dKbh += U dSg
        {
            const bf16x8 ao = frag_rows(sl.dO, PQ, 16 * I, 0, lane);
            const bf16x8 ax = frag_rows(sl.dX, PQ, 16 * I, 0, lane);
            const bf16x8 au = frag_rows(sl.U, PQ, 16 * I, 0, lane);
#pragma unroll
            for (int Ji = 0; Ji < 2; ++Ji) {
                const int J = 2 * half + Ji;
                if (J <= I) dPa[Ji] = mfma32(ao, frag_rows(sl.U, PQ, 16 * J, 0, lane), dPa[Ji]);
            }
#pragma unroll
            for (int cbi = 0; cbi < NBH; ++cbi) {
                const int cb = cb0 + cbi;
                const Frag2 s0{frag_cols(sl.S0h, PD, 0, 16 * cb, lane), frag_cols(sl.S0l, PD, 0, 16 * cb, lane)};
                dQt[cbi] = mfma_ab2(ao, s0, dQt[cbi]);
                dKt[cbi] = mfma_ab2(ax, s0, dKt[cbi]);
                dKbh[cbi] = mfma_ab2(au, Frag2{frag_cols(sl.dSh, PD, 0, 16 * cb, lane),
                                                frag_cols(sl.dSl, PD, 0, 16 * cb, lane)}, dKbh[cbi]);
            }
        }
        __syncthreads();
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) atomicAdd(&sm.dbC[jc + u], dbc[u]);
    // the channel gate again, for E in the last step: loads issued here
    f32x4 gpre[CH ? C * D / 4 / NT : 1];
    if constexpr (CH) gate_load<D, NT>(gpre, gg, gstr, Cc, tid);

    // ---- 8, 11. dP = scale lower(dO U^T) (its diagonal's rounding kept);
    //         dT = lower(dU X^T): dbeta_s += sum_r dT_rs N_rs, dN = dT diag(beta)
#pragma unroll
    for (int Ji = 0; Ji < 2; ++Ji) {
        const int J = 2 * half + Ji;
        const int s = 16 * J + l15;
        const float bs_ = sm.beta[s];
        float part = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = rowof(e);
            const float pv = s <= r ? a.scale * dPa[Ji][e] : 0.f;
            const bf16 pb = (bf16)pv;
            sm.dPb[r * PC + s] = pb;
            if (s == r) sm.pcor[r] = pv - (float)pb;
            const float tv = s <= r ? dTa[Ji][e] : 0.f;
            part += tv * Nreg[Ji][e];
            sm.Pb[r * PC + s] = (bf16)(tv * bs_);
        }
        part = sum_quads(part);
        if (q4 == 0 && J <= I) atomicAdd(&sm.dbeta[s], part);
    }
    __syncthreads();

    // ---- 9, 10. dQt = scale dO S0 + dP Kb;  dKb = dP^T Qt;  dKt = -dX S0
#pragma unroll
    for (int cbi = 0; cbi < NBH; ++cbi) {
        const int cb = cb0 + cbi;
        f32x4 y = zero4();
        dKb[cbi] = zero4();
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            y = mfma32(frag_rows(sm.dPb, PC, 16 * I, 32 * kk, lane), frag_cols(sm.Kb, PD, 32 * kk, 16 * cb, lane), y);
            dKb[cbi] = mfma32(frag_cols(sm.dPb, PC, 32 * kk, 16 * I, lane),
                              frag_cols(sm.Qt, PD, 32 * kk, 16 * cb, lane), dKb[cbi]);
        }
        dQt[cbi] = a.scale * dQt[cbi] + y;
        dKt[cbi] = -dKt[cbi];
        const int j = 16 * cb + l15;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = rowof(e);
            dQt[cbi][e] += sm.pcor[r] * (float)sm.Kb[r * PD + j];
            dKb[cbi][e] += sm.pcor[r] * (float)sm.Qt[r * PD + j];
        }
    }

    // ---- 14. Y = dN N^T (into Tb), dM = -N^T Y;  dbeta_r += sum_s dM_rs A_rs;
    //          dA = strict_lower(diag(beta) dM) (into dPb)
#pragma unroll
    for (int Ji = 0; Ji < 2; ++Ji) {
        const int J = 2 * half + Ji;
        f32x4 y = zero4();
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
            y = mfma32(frag_rows(sm.Pb, PC, 16 * I, 32 * kk, lane), frag_rows(sm.Nb, PC, 16 * J, 32 * kk, lane), y);
        const int s = 16 * J + l15;
#pragma unroll
        for (int e = 0; e < 4; ++e) sm.Tb[rowof(e) * PC + s] = (bf16)y[e];
    }
    __syncthreads();
    float dbr[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int Ji = 0; Ji < 2; ++Ji) {
        const int J = 2 * half + Ji;
        f32x4 m = zero4(), av = zero4();      // A formed again (as in step 2) from Kt, Kb
        if (J <= I) {
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
                m = mfma32(frag_cols(sm.Nb, PC, 32 * kk, 16 * I, lane), frag_cols(sm.Tb, PC, 32 * kk, 16 * J, lane), m);
#pragma unroll
            for (int kk = 0; kk < KD; ++kk)
                av = mfma32(frag_rows(sm.Kt, PD, 16 * I, 32 * kk, lane), frag_rows(sm.Kb, PD, 16 * J, 32 * kk, lane), av);
        }
        const int s = 16 * J + l15;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = rowof(e);
            const float dm = s < r ? -m[e] : 0.f;
            dbr[e] += dm * av[e];
            sm.dPb[r * PC + s] = (bf16)(sm.beta[r] * dm);
        }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const float v = sum_group<16>(dbr[e]);
        if (l15 == 0) atomicAdd(&sm.dbeta[rowof(e)], v);
    }
    __syncthreads();

    // ---- 15. dKt += dA Kb;  dKb += dA^T Kt
#pragma unroll
    for (int cbi = 0; cbi < NBH; ++cbi) {
        const int cb = cb0 + cbi;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            dKt[cbi] = mfma32(frag_rows(sm.dPb, PC, 16 * I, 32 * kk, lane), frag_cols(sm.Kb, PD, 32 * kk, 16 * cb, lane), dKt[cbi]);
            dKb[cbi] = mfma32(frag_cols(sm.dPb, PC, 32 * kk, 16 * I, lane), frag_cols(sm.Kt, PD, 32 * kk, 16 * cb, lane), dKb[cbi]);
        }
    }
    __syncthreads();                           // gated operands no longer read

    // ---- 16. db and h from the bf16 gated operands the products used (so
    //          that the pairs of terms that cancel exactly in dg -- a P or A
    //          entry seen from its row and from its column -- cancel to fp32
    //          accuracy); then E; dq, dk; dg by reverse sums; dbeta
    float *dbf = sm.R.db;                            // db [r][j] (channel gate)
    float *hf = reinterpret_cast<float *>(sm.Tb);    // h [r][j] (channel gate), over Tb..Nb
    float *Ef = reinterpret_cast<float *>(sm.Qt);    // e^b [r][j] (channel gate), over Qt, Kt
    static_assert(sizeof(sm.Tb) + sizeof(sm.Pb) + sizeof(sm.dPb) + sizeof(sm.Nb) >= sizeof(float) * C * D,
                  "h overlay");
    static_assert(sizeof(sm.Qt) + sizeof(sm.Kt) >= sizeof(float) * C * D, "E overlay");
    float rowacc[4] = {0.f, 0.f, 0.f, 0.f}, hacc[4] = {0.f, 0.f, 0.f, 0.f};   // scalar gate
#pragma unroll
    for (int cbi = 0; cbi < NBH; ++cbi) {
        const int cb = cb0 + cbi;
        const int j = 16 * cb + l15;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = rowof(e);
            const float qt = (float)sm.Qt[r * PD + j];
            const float kt = (float)sm.Kt[r * PD + j];
            const float kb = (float)sm.Kb[r * PD + j];
            const float rowsum = dQt[cbi][e] * qt + dKt[cbi][e] * kt - dKb[cbi][e] * kb;
            const float hsum = dKbh[cbi][e] * kb;
            if (CH) {
                dbf[r * D + j] = rowsum;
                hf[r * D + j] = hsum;
            } else {
                rowacc[e] += rowsum;
                hacc[e] += hsum;
            }
        }
    }
    if (!CH) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float v = sum_group<16>(rowacc[e]);
            const float hv = sum_group<16>(hacc[e]);
            if (l15 == 0) {
                atomicAdd(&sm.dbrow[rowof(e)], v);
                atomicAdd(&sm.hrow[rowof(e)], hv);
            }
        }
    }
    __syncthreads();                           // Qt, Kt no longer read
    float *ptot = reinterpret_cast<float *>(sm.R.stage) + C * D;   // 2 NT floats past db
    static_assert(sizeof(sm.R) >= sizeof(float) * (C * D + 2 * NT), "part sums");
    if constexpr (CH) gate_sums_from<D, NT>(Ef, ptot, gpre, tid);   // b, over Qt and Kt
#pragma unroll
    for (int cbi = 0; cbi < NBH; ++cbi) {
        const int cb = cb0 + cbi;
        const int j = 16 * cb + l15;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = rowof(e);
            const float E = ex(CH ? Ef[r * D + j] : sm.bs[r]);
            const float Ei = __builtin_amdgcn_rcpf(E);
            if (r < Cc) {
                const size_t o = ((tok0 + r) * a.H + h) * D + j;
                a.dq[o] = dQt[cbi][e] * E;
                a.dk[o] = dKt[cbi][e] * E + (dKb[cbi][e] + dKbh[cbi][e]) * Ei;
            }
        }
    }
    __syncthreads();
    if (CH) {
        // dg_s = sum_{r >= s} db_r + db_C + sum_{r < s} h_r per channel: NT / D
        // parts of the rows per channel, each taken by one thread, with the
        // sums of the other parts as offsets
        constexpr int NH = NT / D, RH = C / NH;
        const int j = tid % D, part = tid / D;
        float hs = 0.f, ds = 0.f;
#pragma unroll
        for (int u = 0; u < RH; ++u) {
            hs += hf[(part * RH + u) * D + j];
            ds += dbf[(part * RH + u) * D + j];
        }
        ptot[part * D + j] = hs;
        ptot[(NH + part) * D + j] = ds;
        __syncthreads();
        float pre = 0.f, run = sm.dbC[j];
        for (int q = 0; q < part; ++q) pre += ptot[q * D + j];
        for (int q = NH - 1; q > part; --q) run += ptot[(NH + q) * D + j];
        float hx[RH];
#pragma unroll
        for (int u = 0; u < RH; ++u) {
            hx[u] = pre;
            pre += hf[(part * RH + u) * D + j];
        }
#pragma unroll
        for (int u = RH - 1; u >= 0; --u) {
            const int r = part * RH + u;
            run += dbf[r * D + j];
            if (r < Cc) a.dg[(tok0 + r) * a.H * D + (size_t)h * D + j] = run + hx[u];
        }
    } else if (w == 0) {
        // scalar gate: db_C summed over channels; lane 63 - s takes row s:
        // the suffix sum of db over rows >= s, the prefix of h over rows < s
        float tot = 0.f;
        for (int j = lane; j < D; j += 64) tot += sm.dbC[j];
        tot = sum_quads(sum_group<16>(tot));
        const float hx = wave_prefix_sum(lane > 0 ? sm.hrow[lane - 1] : 0.f);   // row lane
        const int s = C - 1 - lane;
        const float suf = wave_prefix_sum(sm.dbrow[s]);
        const float hs = __shfl(hx, s);
        if (s < Cc) a.dg[(tok0 + s) * a.H + h] = tot + suf + hs;
    }
    if (tid < Cc) a.dbeta[(tok0 + tid) * a.H + h] = sm.dbeta[tid];
}

// ===========================================================================
// adjoint_chain_kernel: the state gradient chunk by chunk, in reverse.  From
// the chunked form, with dSg = dS_C Diag(e^{b_C}),
//     dU = Kb dSg^T + scale P^T dO,    dS_0 = dSg + scale dO^T Qt - dU^T W,
// W = T Kt; the rows of dS (value index) never mix, so one workgroup owns a
// BVA-row slice of one (sequence, head) and walks its chunks from the last,
// dS in fp32 accumulators (each wave a quarter of the key columns), staging
// each chunk's ChainRec and dO slice in LDS (the next chunk's loaded into
// registers meanwhile).  It stores every chunk's dS_C and finally dS_0
// (dh0).  Two workgroups fit on a CU: when there are more (sequence, head,
// slice) units than CUs, that doubles the chunks in flight.
// ===========================================================================
constexpr int BVA = 16;     // value rows per chain workgroup (76.8 KB of LDS at D = 128: two per CU)
constexpr int NVB = BVA / 16, NDP = BVA / 8;   // 16-row value blocks; 8-wide dO pieces per row

template <int D> struct ChainSmem {
    static constexpr int PD = D + 8, PV = BVA + 8;
    alignas(16) bf16 Qt[C * PD];
    alignas(16) bf16 Kb[C * PD];
    alignas(16) bf16 W[C * PD];
    alignas(16) bf16 P[C * PC];
    alignas(16) float eC[D];
    alignas(16) bf16 dO[C * PV];      // [r][i]
    alignas(16) bf16 dSh[BVA * PD];   // dSg as hi + lo bf16, [i][j]
    alignas(16) bf16 dSl[BVA * PD];
    alignas(16) bf16 dU[C * PV];      // [r][i]
};

template <int D>
__global__ __launch_bounds__(256) void adjoint_chain_kernel(BwdArgs a) {
    using Sm = ChainSmem<D>;
    using R = ChainRec<D>;
    constexpr int PD = Sm::PD, PV = Sm::PV;
    constexpr int NTL = D / BVA;
    constexpr int CB = D * NVB / 64;  // key blocks per wave: BVA x D of dS over 4 waves
    __shared__ Sm sm;
    // the value slices of one (sequence, head) on one XCD
    const int bid = blockIdx.x;
    const int xcd = bid & 7, jj = bid >> 3;
    const int tile = jj % NTL;
    const int unit = (jj / NTL) * 8 + xcd;
    if (unit >= a.B * a.H) return;
    const int b = unit / a.H, h = unit - b * a.H;     // sequence b
    long long seq0, len, cb;                          // first token, length, first global chunk
    if (a.cu_seqlens) {
        seq0 = a.cu_seqlens[b];
        len = a.cu_seqlens[b + 1] - seq0;
        cb = a.chunk_base[b];
    } else {
        seq0 = (long long)b * a.T;
        len = a.T;
        cb = (long long)b * a.nc;
    }
    const int nch = (int)((len + C - 1) / C);
    const int i0 = tile * BVA;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l15 = lane & 15, q4 = lane >> 4;
    const int ib = w % NVB, jb0 = CB * (w / NVB);
    const size_t rowD = (size_t)a.H * D;
    const size_t bh = (size_t)b * a.H + h;

    // dS tiles: element e of tile t = row i0 + 16 ib + 4 q4 + e, column 16 (jb0 + t) + l15
    f32x4 dS[CB];
#pragma unroll
    for (int t = 0; t < CB; ++t) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const size_t o = bh * D * D + (size_t)(i0 + 16 * ib + 4 * q4 + e) * D + 16 * (jb0 + t) + l15;
            dS[t][e] = a.dht ? a.dht[o] : 0.f;
        }
    }
    // the next chunk's record and dO slice, in registers while this one is
    // worked on
    constexpr int NR = C * D / 8 / 256, NP = C * C / 8 / 256;
    bf16x8 rq[NR], rk[NR], rw[NR], rp[NP], rdo;
    float rec_ = 0.f;
    auto fetch = [&](int c) {
        const char *rec = static_cast<const char *>(a.recs) + ((size_t)(cb + c) * a.H + h) * R::BYTES;
#pragma unroll
        for (int it = 0; it < NR; ++it) {
            const int p = it * 256 + tid, r = p / (D / 8), j = 8 * (p % (D / 8));
            rq[it] = *reinterpret_cast<const bf16x8 *>(rec + R::QT + 2 * (r * D + j));
            rk[it] = *reinterpret_cast<const bf16x8 *>(rec + R::KB + 2 * (r * D + j));
            rw[it] = *reinterpret_cast<const bf16x8 *>(rec + R::W + 2 * (r * D + j));
        }
#pragma unroll
        for (int it = 0; it < NP; ++it) {
            const int p = it * 256 + tid, r = p / (C / 8), sc = 8 * (p % (C / 8));
            rp[it] = *reinterpret_cast<const bf16x8 *>(rec + R::P + 2 * (r * C + sc));
        }
        if (tid < D) rec_ = reinterpret_cast<const float *>(rec + R::EC)[tid];
        const int t0 = c * C, r = tid / NDP;                // 64 rows x NDP pieces of 8
        rdo = bf16x8{};
        if (tid < C * NDP && r < len - t0)
            rdo = *reinterpret_cast<const bf16x8 *>(static_cast<const bf16 *>(a.dout) +
                                                    ((size_t)(seq0 + t0 + r) * a.H + h) * D + i0 + 8 * (tid % NDP));
    };
    static_assert(C * D / 8 % 256 == 0 && C * C / 8 % 256 == 0, "record pieces per thread");
    if (nch > 0) fetch(nch - 1);
    for (int c = nch - 1; c >= 0; --c) {
        // dS_C of chunk c
        float *dsc = a.dstates + ((size_t)(cb + c) * a.H + h) * D * D;
#pragma unroll
        for (int t = 0; t < CB; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                dsc[(size_t)(i0 + 16 * ib + 4 * q4 + e) * D + 16 * (jb0 + t) + l15] = dS[t][e];
        // stage the record and the dO slice (loaded during the previous chunk)
#pragma unroll
        for (int it = 0; it < NR; ++it) {
            const int p = it * 256 + tid, r = p / (D / 8), j = 8 * (p % (D / 8));
            *reinterpret_cast<bf16x8 *>(&sm.Qt[r * PD + j]) = rq[it];
            *reinterpret_cast<bf16x8 *>(&sm.Kb[r * PD + j]) = rk[it];
            *reinterpret_cast<bf16x8 *>(&sm.W[r * PD + j]) = rw[it];
        }
#pragma unroll
        for (int it = 0; it < NP; ++it) {
            const int p = it * 256 + tid, r = p / (C / 8), sc = 8 * (p % (C / 8));
            *reinterpret_cast<bf16x8 *>(&sm.P[r * PC + sc]) = rp[it];
        }
        if (tid < D) sm.eC[tid] = rec_;
        if (tid < C * NDP) *reinterpret_cast<bf16x8 *>(&sm.dO[(tid / NDP) * PV + 8 * (tid % NDP)]) = rdo;
        if (c > 0) fetch(c - 1);
        __syncthreads();
        // dSg = dS e^{b_C} as hi + lo bf16
#pragma unroll
        for (int t = 0; t < CB; ++t) {
            const int j = 16 * (jb0 + t) + l15;
            const float ec = sm.eC[j];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float v = dS[t][e] * ec;
                const bf16 hi = (bf16)v;
                const int ii = 16 * ib + 4 * q4 + e;
                sm.dSh[ii * PD + j] = hi;
                sm.dSl[ii * PD + j] = (bf16)(v - (float)hi);
            }
        }
        __syncthreads();
        // dU = Kb dSg^T + scale P^T dO: wave w takes row block w, both value blocks
#pragma unroll
        for (int vb = 0; vb < NVB; ++vb) {
            f32x4 x = {0.f, 0.f, 0.f, 0.f}, y = x;
#pragma unroll
            for (int kk = 0; kk < D / 32; ++kk) {
                const bf16x8 kf = frag_rows(sm.Kb, PD, 16 * w, 32 * kk, lane);
                x = mfma32(kf, frag_rows(sm.dSh, PD, 16 * vb, 32 * kk, lane), x);
                x = mfma32(kf, frag_rows(sm.dSl, PD, 16 * vb, 32 * kk, lane), x);
            }
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
                y = mfma32(frag_cols(sm.P, PC, 32 * kk, 16 * w, lane), frag_cols(sm.dO, PV, 32 * kk, 16 * vb, lane), y);
            const int i = 16 * vb + l15;
#pragma unroll
            for (int e = 0; e < 4; ++e) sm.dU[(16 * w + 4 * q4 + e) * PV + i] = (bf16)(x[e] + a.scale * y[e]);
        }
        __syncthreads();
        // dS_0 = dSg + scale dO^T Qt - dU^T W
#pragma unroll
        for (int t = 0; t < CB; ++t) {
            const int jb = jb0 + t;
            f32x4 x = {0.f, 0.f, 0.f, 0.f}, y = x;
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                x = mfma32(frag_cols(sm.dO, PV, 32 * kk, 16 * ib, lane), frag_cols(sm.Qt, PD, 32 * kk, 16 * jb, lane), x);
                y = mfma32(frag_cols(sm.dU, PV, 32 * kk, 16 * ib, lane), frag_cols(sm.W, PD, 32 * kk, 16 * jb, lane), y);
            }
            const float ec = sm.eC[16 * jb + l15];
            dS[t] = dS[t] * ec + a.scale * x - y;
        }
        __syncthreads();                       // before the next chunk's staging
    }
    if (a.dh0) {
#pragma unroll
        for (int t = 0; t < CB; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                a.dh0[bh * D * D + (size_t)(i0 + 16 * ib + 4 * q4 + e) * D + 16 * (jb0 + t) + l15] = dS[t][e];
    }
}

// dst = src, or zeros without src (a kernel, so that the call can be
// captured in a graph)
__global__ __launch_bounds__(256) void copy_or_zero_kernel(float *dst, const float *src, size_t n) {
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) dst[i] = src ? src[i] : 0.f;
}

}  // namespace

hipError_t launch_copy_or_zero(float *dst, const float *src, size_t n, hipStream_t s) {
    if (n == 0) return hipSuccess;
    const size_t blocks = (n + 255) / 256;
    if (blocks >= (1ULL << 31)) return hipErrorInvalidValue;
    hipLaunchKernelGGL(copy_or_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, s, dst, src, n);
    return hipGetLastError();
}

size_t backward_record_bytes(int D) {
    return D == 128 ? ChainRec<128>::BYTES : ChainRec<64>::BYTES;
}

// ===========================================================================
// Pairs beyond the chunk factorisation
// ===========================================================================
// The chunk-local gradients factor each chunk from its first token
// (k e^{-b} inside a chunk), which holds while no channel decays by more
// than e^80 over a chunk.  The forward pass marks the (sequence, head) pairs
// where one does (unit_wide); every gradient of such a pair is recomputed
// here, exactly, by the adjoint of the token recurrence in fp32, from the
// chunk-entering states the forward stored (the chunked forward itself is
// exact for every gate).  Per value row i of the state (rows never mix),
// with s = s_{t-1}, u = a_t (.) s, e = v_ti - u.k_t,
// s_t = u + beta_t e k_t and o_ti = scale s_t.q_t, and G the gradient of
// s_t through everything after token t:
//     G' = G + scale do_ti q_t           dq_t += scale do_ti s_t
//     dv_ti = beta_t (G'.k_t)            dbeta_t += e (G'.k_t)
//     dk_t += beta_t e G' - beta_t (G'.k_t) u
//     du = G' - beta_t (G'.k_t) k_t      dg_t += du (.) u   (summed over
//     G <- a_t (.) du                    channels for the scalar gate)
// so dq, dk, dg and dbeta are sums over the rows and dv, dh0 are row-local.
// A workgroup (16 waves) takes 64 rows of one pair, 16 lanes to a row with
// D/16 columns each; a chunk is walked backwards in blocks of kWideBlk
// tokens and those in sub-blocks of kWideSub, the block's entering state
// recomputed forward from the chunk's stored state and each sub-block's
// from the block's (kWideSub token states stay in registers).  The
// column sums over the 64 rows go through LDS; at D = 128 the two
// workgroups of a pair add theirs into outputs the zeroing kernel cleared
// -- two fp32 additions onto zero, whose result does not depend on their
// order, so the gradients are the same on every run.
constexpr int kWideSub = 4;    // token states a lane keeps at once
constexpr int kWideBlk = 16;   // tokens whose entering state is kept

template <int D, bool CH> struct WideSmem {
    static constexpr int NA = CH ? D : 1;
    static constexpr int NV = CH ? 3 : 2;          // column sums: dq, dk (, dg)
    alignas(16) float a[C * NA];                    // e^g per token (and channel)
    alignas(16) bf16 k[C * D], q[C * D];
    alignas(16) float v[C * 64], dout[C * 64];      // the workgroup's 64 value rows
    alignas(16) float beta[C];
    alignas(16) float red[2][16][NV * D];           // per-wave column sums, two tokens
    alignas(16) float reds[2][16][2];               // per-wave dbeta (, scalar dg)
};

template <int VPL>
__device__ inline void lds_row(const bf16 *p, float (&x)[VPL]) {
    if constexpr (VPL == 8) {
        const bf16x8 r = *reinterpret_cast<const bf16x8 *>(p);
#pragma unroll
        for (int j = 0; j < 8; ++j) x[j] = (float)r[j];
    } else {
        const bf16x4 r = *reinterpret_cast<const bf16x4 *>(p);
#pragma unroll
        for (int j = 0; j < 4; ++j) x[j] = (float)r[j];
    }
}

template <int D, bool CH>
__device__ inline void wide_gate(const WideSmem<D, CH> &sm, int t, int j0, float (&at)[D / 16]) {
#pragma unroll
    for (int j = 0; j < D / 16; ++j) at[j] = CH ? sm.a[t * D + j0 + j] : sm.a[t];
}

// one token forward on a lane's part of a row: s <- s_t; returns e
template <int D, bool CH>
__device__ inline float wide_fwd(const WideSmem<D, CH> &sm, float (&s)[D / 16], int t, int rl,
                                 int j0) {
    constexpr int VPL = D / 16;
    float kk[VPL], at[VPL];
    lds_row<VPL>(sm.k + t * D + j0, kk);
    wide_gate<D, CH>(sm, t, j0, at);
    float kd = 0.f;
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
        s[j] *= at[j];
        kd += s[j] * kk[j];
    }
    kd = sum_group<16>(kd);
    const float e = sm.v[t * 64 + rl] - kd;
    const float be = sm.beta[t] * e;
#pragma unroll
    for (int j = 0; j < VPL; ++j) s[j] += be * kk[j];
    return e;
}

template <int D, bool CH>
__global__ __launch_bounds__(1024) void wide_backward_kernel(BwdArgs a) {
    constexpr int P = D / 64;
    constexpr int VPL = D / 16;
    constexpr int NV = WideSmem<D, CH>::NV;
    __shared__ WideSmem<D, CH> sm;
    const long long unit = blockIdx.x / P;
    const int part = blockIdx.x % P;
    if (unit >= (long long)a.B * a.H || !a.unit_wide[unit]) return;
    const int n = (int)(unit / a.H), h = (int)(unit % a.H);
    long long t0, len;
    if (a.cu_seqlens) {
        t0 = a.cu_seqlens[n];
        len = a.cu_seqlens[n + 1] - t0;
    } else {
        t0 = (long long)n * a.T;
        len = a.T;
    }
    const long long cb = a.cu_seqlens ? (long long)a.chunk_base[n] : (long long)n * a.nc;
    const int nch = (int)((len + C - 1) / C);
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    const int rl = 4 * w + (lane >> 4);            // row within the workgroup's 64
    const int r = 64 * part + rl;                  // value row of the state
    const int j0 = VPL * (lane & 15);
    const size_t DD = (size_t)D * D;
    const bf16 *qg = static_cast<const bf16 *>(a.q), *kg = static_cast<const bf16 *>(a.k);
    const bf16 *vg = static_cast<const bf16 *>(a.v), *dog = static_cast<const bf16 *>(a.dout);
    float G[VPL];
#pragma unroll
    for (int j = 0; j < VPL; ++j)
        G[j] = a.dht ? a.dht[(size_t)unit * DD + (size_t)r * D + j0 + j] : 0.f;
    int par = 0;
    for (int c = nch - 1; c >= 0; --c) {
        const int L = (int)(len - (long long)C * c < C ? len - (long long)C * c : C);
        const long long tc = t0 + (long long)C * c;
        __syncthreads();                           // the previous chunk's reads are done
        // stage the chunk: k, q rows (bf16), e^g, this workgroup's v and do
        // columns (fp32), beta; tokens past L as zeros
        for (int x = tid; x < C * D / 8; x += 1024) {
            const int t = x / (D / 8), c8 = x % (D / 8);
            bf16x8 kv = {}, qv = {};
            if (t < L) {
                const size_t o = ((size_t)(tc + t) * a.H + h) * D + 8 * c8;
                kv = *reinterpret_cast<const bf16x8 *>(kg + o);
                qv = *reinterpret_cast<const bf16x8 *>(qg + o);
            }
            *reinterpret_cast<bf16x8 *>(sm.k + t * D + 8 * c8) = kv;
            *reinterpret_cast<bf16x8 *>(sm.q + t * D + 8 * c8) = qv;
        }
        if (CH) {
            for (int x = tid; x < C * D / 4; x += 1024) {
                const int t = x / (D / 4), c4 = x % (D / 4);
                f32x4 gv = {0.f, 0.f, 0.f, 0.f};
                if (t < L)
                    gv = *reinterpret_cast<const f32x4 *>(a.g + ((size_t)(tc + t) * a.H + h) * D + 4 * c4);
                f32x4 av;
#pragma unroll
                for (int u = 0; u < 4; ++u) av[u] = ex(__builtin_fmaxf(gv[u], kGateFloor));
                *reinterpret_cast<f32x4 *>(sm.a + t * D + 4 * c4) = av;
            }
        } else if (tid < C) {
            sm.a[tid] = tid < L ? ex(__builtin_fmaxf(a.g[(size_t)(tc + tid) * a.H + h], kGateFloor)) : 1.f;
        }
        for (int x = tid; x < C * 8; x += 1024) {  // 64 rows = 8 pieces of 8 per token
            const int t = x >> 3, c8 = x & 7;
            bf16x8 vv = {}, dv = {};
            if (t < L) {
                const size_t o = ((size_t)(tc + t) * a.H + h) * D + 64 * part + 8 * c8;
                vv = *reinterpret_cast<const bf16x8 *>(vg + o);
                dv = *reinterpret_cast<const bf16x8 *>(dog + o);
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                sm.v[t * 64 + 8 * c8 + u] = (float)vv[u];
                sm.dout[t * 64 + 8 * c8 + u] = (float)dv[u] * a.scale;
            }
        }
        if (tid < C) sm.beta[tid] = tid < L ? a.beta[(size_t)(tc + tid) * a.H + h] : 0.f;
        __syncthreads();
        // the chunk in blocks of kWideBlk tokens, last first: a block's
        // entering state forward from the chunk's stored one, then the
        // block in sub-blocks of kWideSub, each entered from the block's
        // state (the same steps in the same order as from the chunk start)
        const float *sc = a.states + ((size_t)(cb + c) * a.H + h) * DD;   // uniform
        for (int tb = (L - 1) / kWideBlk * kWideBlk; tb >= 0; tb -= kWideBlk) {
          float sbk[VPL];
#pragma unroll
          for (int j = 0; j < VPL; ++j) sbk[j] = sc[r * D + j0 + j];
          for (int t = 0; t < tb; ++t) wide_fwd<D, CH>(sm, sbk, t, rl, j0);
          const int Lb = L - tb < kWideBlk ? L - tb : kWideBlk;
          for (int sb = (Lb - 1) / kWideSub; sb >= 0; --sb) {
            float s[VPL];
#pragma unroll
            for (int j = 0; j < VPL; ++j) s[j] = sbk[j];
            for (int t = tb; t < tb + kWideSub * sb; ++t) wide_fwd<D, CH>(sm, s, t, rl, j0);
            const int nt = Lb - kWideSub * sb < kWideSub ? Lb - kWideSub * sb : kWideSub;
            float st[kWideSub][VPL], e[kWideSub];
#pragma unroll
            for (int u = 0; u < kWideSub; ++u) {
                if (u < nt) {
#pragma unroll
                    for (int j = 0; j < VPL; ++j) st[u][j] = s[j];
                    e[u] = wide_fwd<D, CH>(sm, s, tb + kWideSub * sb + u, rl, j0);
                }
            }
#pragma unroll
            for (int u = kWideSub - 1; u >= 0; --u) {
                if (u >= nt) continue;
                const int t = tb + kWideSub * sb + u;
                const size_t row = (size_t)(tc + t) * a.H + h;
                float kk[VPL], qq[VPL], at[VPL];
                lds_row<VPL>(sm.k + t * D + j0, kk);
                lds_row<VPL>(sm.q + t * D + j0, qq);
                wide_gate<D, CH>(sm, t, j0, at);
                const float b = sm.beta[t], dor = sm.dout[t * 64 + rl], eu = e[u];
                // each column sum is taken over the wave's four rows and
                // stored as soon as it is formed (few values live at once)
                float uu[VPL], gk = 0.f;
#pragma unroll
                for (int j = 0; j < VPL; ++j) {
                    uu[j] = at[j] * st[u][j];
                    const float pq = swap_sum32(swap_sum16(dor * (uu[j] + b * eu * kk[j])));
                    if (lane < 16) sm.red[par][w][j0 + j] = pq;       // scale do_ti s_t
                    G[j] += dor * qq[j];
                    gk += G[j] * kk[j];
                }
                gk = sum_group<16>(gk);
                if ((lane & 15) == 0) a.dv[row * D + r] = b * gk;
                const float de = b * gk, be = b * eu;
                float pgs = 0.f;
#pragma unroll
                for (int j = 0; j < VPL; ++j) {
                    const float pk = swap_sum32(swap_sum16(be * G[j] - de * uu[j]));
                    if (lane < 16) sm.red[par][w][D + j0 + j] = pk;
                    const float du = G[j] - de * kk[j];
                    if (CH) {
                        const float pg = swap_sum32(swap_sum16(du * uu[j]));
                        if (lane < 16) sm.red[par][w][2 * D + j0 + j] = pg;
                    } else {
                        pgs += du * uu[j];
                    }
                    G[j] = at[j] * du;
                }
                const float pb = swap_sum32(swap_sum16(eu * gk));
                if (!CH) pgs = swap_sum32(swap_sum16(sum_group<16>(pgs)));
                if (lane == 0) {
                    sm.reds[par][w][0] = pb;
                    sm.reds[par][w][1] = pgs;
                }
                __syncthreads();
                if (tid < NV * D) {
                    const int comp = tid / D, j = tid % D;
                    float sum = 0.f;
#pragma unroll
                    for (int x = 0; x < 16; ++x) sum += sm.red[par][x][tid];
                    float *dst = comp == 0 ? a.dq : comp == 1 ? a.dk : a.dg;
                    atomicAdd(dst + row * D + j, sum);
                } else if (tid < NV * D + (CH ? 1 : 2)) {
                    const int comp = tid - NV * D;
                    float sum = 0.f;
#pragma unroll
                    for (int x = 0; x < 16; ++x) sum += sm.reds[par][x][comp];
                    atomicAdd(comp == 0 ? a.dbeta + row : a.dg + row, sum);
                }
                par ^= 1;
            }
          }
        }
    }
    if (a.dh0) {
#pragma unroll
        for (int j = 0; j < VPL; ++j) a.dh0[(size_t)unit * DD + (size_t)r * D + j0 + j] = G[j];
    }
}

// Clears dq, dk, dg and dbeta of the marked pairs (the wide kernel adds into
// them).  One workgroup per (pair, part of its tokens).
constexpr int kZeroParts = 16;
template <int D>
__global__ __launch_bounds__(256) void wide_zero_kernel(BwdArgs a) {
    const long long unit = blockIdx.x / kZeroParts;
    const int part = blockIdx.x % kZeroParts;
    if (unit >= (long long)a.B * a.H || !a.unit_wide[unit]) return;
    const int n = (int)(unit / a.H), h = (int)(unit % a.H);
    long long t0, len;
    if (a.cu_seqlens) {
        t0 = a.cu_seqlens[n];
        len = a.cu_seqlens[n + 1] - t0;
    } else {
        t0 = (long long)n * a.T;
        len = a.T;
    }
    const long long per = (len + kZeroParts - 1) / kZeroParts;
    const long long r0 = part * per, r1 = r0 + per < len ? r0 + per : len;
    for (long long idx = r0 * D + threadIdx.x; idx < r1 * D; idx += 256) {
        const long long t = t0 + idx / D;
        const int j = (int)(idx % D);
        const size_t o = ((size_t)t * a.H + h) * D + j;
        a.dq[o] = 0.f;
        a.dk[o] = 0.f;
        if (a.channel_gate) a.dg[o] = 0.f;
        else if (j == 0) a.dg[(size_t)t * a.H + h] = 0.f;
        if (j == 0) a.dbeta[(size_t)t * a.H + h] = 0.f;
    }
}

hipError_t launch_backward(int D, const BwdArgs &a, hipStream_t s) {
    const long long heads = (long long)a.B * a.H;
    if (heads <= 0 || a.chunks <= 0) return hipSuccess;
    const long long chain_blocks = ((heads + 7) / 8) * 8 * (D / BVA);
    const long long chunk_blocks = a.chunks * a.H;
    if (chain_blocks >= (1LL << 31) || chunk_blocks >= (1LL << 31)) return hipErrorInvalidValue;
    dim3 gr((unsigned)chain_blocks), gc((unsigned)chunk_blocks), blk(256), blk8(512);
    if (D == 128) {
        if (a.channel_gate) hipLaunchKernelGGL((chunk_grad_kernel<128, true, true>), gc, blk8, 0, s, a);
        else                hipLaunchKernelGGL((chunk_grad_kernel<128, false, true>), gc, blk8, 0, s, a);
        hipLaunchKernelGGL(adjoint_chain_kernel<128>, gr, blk, 0, s, a);
        if (a.channel_gate) hipLaunchKernelGGL((chunk_grad_kernel<128, true, false>), gc, blk8, 0, s, a);
        else                hipLaunchKernelGGL((chunk_grad_kernel<128, false, false>), gc, blk8, 0, s, a);
    } else {
        if (a.channel_gate) hipLaunchKernelGGL((chunk_grad_kernel<64, true, true>), gc, blk8, 0, s, a);
        else                hipLaunchKernelGGL((chunk_grad_kernel<64, false, true>), gc, blk8, 0, s, a);
        hipLaunchKernelGGL(adjoint_chain_kernel<64>, gr, blk, 0, s, a);
        if (a.channel_gate) hipLaunchKernelGGL((chunk_grad_kernel<64, true, false>), gc, blk8, 0, s, a);
        else                hipLaunchKernelGGL((chunk_grad_kernel<64, false, false>), gc, blk8, 0, s, a);
    }
    if (a.unit_wide) {
        // the marked pairs again, exactly: their sums cleared, then the
        // token-level adjoint
        if (heads * kZeroParts >= (1LL << 31) || heads * (D / 64) >= (1LL << 31))
            return hipErrorInvalidValue;
        dim3 gz((unsigned)(heads * kZeroParts)), gw((unsigned)(heads * (D / 64)));
        if (D == 128) {
            hipLaunchKernelGGL(wide_zero_kernel<128>, gz, dim3(256), 0, s, a);
            if (a.channel_gate) hipLaunchKernelGGL((wide_backward_kernel<128, true>), gw, dim3(1024), 0, s, a);
            else                hipLaunchKernelGGL((wide_backward_kernel<128, false>), gw, dim3(1024), 0, s, a);
        } else {
            hipLaunchKernelGGL(wide_zero_kernel<64>, gz, dim3(256), 0, s, a);
            if (a.channel_gate) hipLaunchKernelGGL((wide_backward_kernel<64, true>), gw, dim3(1024), 0, s, a);
            else                hipLaunchKernelGGL((wide_backward_kernel<64, false>), gw, dim3(1024), 0, s, a);
        }
    }
    return hipGetLastError();
}

}  // namespace gdr
