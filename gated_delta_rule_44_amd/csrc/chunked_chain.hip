// chunked_chain.hip -- chunked prefill of the gated delta rule with the
// state recurrence on dedicated waves (scalar gate, Gated DeltaNet).
//
// Chunked form ("Super Apriel: One Checkpoint, Many Speeds", gist.science
// summary 2a, for the recurrence; the reorganisation into chunks is derived
// in chunked.hip).  For a chunk of C = 64 tokens entering with state S (Dv x
// Dk), b_r the in-chunk cumulative log gate and beta_r the write strength:
//     A[r][s] = e^{b_r - b_s} k_r.k_s (s < r),  P[r][s] = e^{b_r - b_s} q_r.k_s
//     (s <= r),  L = diag(beta) A,  T = (I + L)^{-1} diag(beta)
//     X = V - diag(e^b) K S^T,   U = T X
//     O = scale (diag(e^b) Q S^T + P U)
//     S^T <- e^{b_C} S^T + K^T diag(e^{b_C - b}) U
//
// Work split.  The only dependency from chunk to chunk is the state, through
// X, U and the update.  Two "chain" waves each own 16 of the workgroup's 32
// value columns and keep their slice of S^T (Dk x 16, fp32) in accumulator
// registers for the whole sequence; they do nothing but X, U and the update,
// and publish S^T and U (as bf16 MFMA operands) for the output waves.  A
// single wave streams LDS at only a fraction of the CU's bandwidth, so
// everything else is spread over the other six waves, one or two chunks
// behind or ahead: the A and P blocks and the inverse T (waves 2, 3, 6, 7),
// the outputs O (waves 4, 5), staging of q, k, v into LDS and the gate
// prefix sums (waves 4..7).
//
// Operands that come from accumulator registers (S^T, X, U) feed the next
// MFMA directly in the paired k order of device_util.h.  q and k rows are
// kept in LDS in that same order (within each 32-column block, columns
// 4m..4m+3 and 16+4m..16+4m+3 are adjacent), so a paired A operand is one
// 16-byte read; the A and P products take both operands from these rows, so
// the order cancels there.  T and P live in LDS as 16x16 blocks in
// accumulator order, transposed (block (i, j) holds T_ij^T), which is the A
// operand of U = T X in the paired order.
//
// T by blocks.  Each diagonal block Y_bb = (I + L_bb)^{-1} is the finite
// series (I - M)(I + M^2)(I + M^4)(I + M^8) of its strictly lower 16x16 block
// M (M^16 = 0); the powers and products are 16x16x16 MFMAs, computed in
// both orientations because an MFMA takes its A operand transposed relative
// to the accumulator layout.  Off the diagonal, block forward substitution
// Y_ij = -Y_ii sum_{k=j}^{i-1} L_ik Y_kj; T = Y diag(beta).
//
// Two barriers per chunk; iteration c of the loop:
//   alpha: chain: X (chunk c) | waves 2,3,6,7: T off the diagonal (c), A and
//          P blocks (c+1) | waves 4,5: O (c-1), diag(e^b) Q S^T (c)
//   beta:  chain: U, state update (c) | waves 2,3,6,7: diagonal blocks of T
//          (c+1) | waves 4..7: q, k, v of chunk c+2 into LDS, gate prefix
//          sums (c+2), global loads of chunk c+3
#include "gdr_internal.h"
#include "device_util.h"

namespace gdr {
namespace {

constexpr int C = 64;        // chunk length
constexpr int NW = 8;        // waves per workgroup
constexpr int NT = NW * 64;  // threads per workgroup
constexpr int BV = 32;       // value columns per workgroup

__device__ inline int tri(int i, int j) { return i * (i + 1) / 2 + j; }   // block (i >= j)
__device__ inline int ltri(int i, int j) { return i * (i - 1) / 2 + j; }  // block (i > j)

template <int D> struct ChainSmem {
    // q and k rows in paired column order; a row stride of 8 x odd dwords
    // keeps the 16-byte row fragment reads free of bank conflicts (and halves
    // those of the transpose reads of k, against 4 x odd)
    static constexpr int PD = D + 16;
    static constexpr int KD = D / 32;
    // v slice rows [r][i]; a stride of 24 dwords puts the 8 rows that one
    // transpose load touches per half-wave on disjoint banks
    static constexpr int PV = BV + 16;
    alignas(16) bf16 Q[2][C * PD];      // by chunk parity
    alignas(16) bf16 K[3][C * PD];      // by chunk mod 3
    alignas(16) bf16 V[2][C * PV];      // by chunk parity
    alignas(16) bf16 TT[2][10 * 256];   // T_ij^T, i >= j, by chunk parity
    alignas(16) bf16 PT[3][10 * 256];   // P_ij^T, i >= j, by chunk mod 3
    alignas(16) bf16 LT[2][6 * 256];    // L_ij^T, i > j, by chunk parity
    alignas(16) bf16 YD[4][2][256];     // Y_bb and Y_bb^T of the next chunk
    alignas(16) bf16x8 SB[2][KD][64];   // S^T as paired B operands, per chain wave
    alignas(16) bf16x8 UB[2][2][64];    // U as paired B operands, per chain wave
    alignas(16) float fb[3][C];         // b_r, by chunk mod 3
    alignas(16) float feb[3][C];        // e^{b_r}
    alignas(16) float fhs[3][C];        // e^{b_C - b_r}
    alignas(16) float fbeta[3][C];      // beta_r
    alignas(16) float fgc[3][4];        // e^{b_C}
};

template <int D>
__global__ __launch_bounds__(NT, 1) void chain_kernel(PrefillArgs a) {
    using Sm = ChainSmem<D>;
    constexpr int PD = Sm::PD;
    constexpr int PV = Sm::PV;
    constexpr int NTILE = D / BV;
    constexpr int KD = Sm::KD;          // paired k steps over Dk
    constexpr int KS = D / 16;          // 16-row blocks of S^T
    constexpr int CG = D / 8;           // 16-byte pieces per q or k row
    constexpr int NPC = C * CG / 256;   // pieces per staging thread and matrix
    static_assert(NPC >= 1 && (C * CG) % 256 == 0, "staging layout");
    __shared__ Sm sm;

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
    const unsigned rowb = (unsigned)(tokstride * 2);   // bytes between tokens
    const bf16 *qg = static_cast<const bf16 *>(a.q) + (size_t)h * D;
    const bf16 *kg = static_cast<const bf16 *>(a.k) + (size_t)h * D;
    const bf16 *vg = static_cast<const bf16 *>(a.v) + (size_t)h * D + i0;
    bf16 *og = static_cast<bf16 *>(a.o) + (size_t)h * D + i0;
    const long long nch = (t1 - t0 + C - 1) / C;

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int l15 = lane & 15, q4 = lane >> 4;

    // rows of chunk c that exist (0 past the end and for the placeholder
    // chunks c < 0 of the pipeline start); buffer extents cover just these,
    // so loads of other rows return zeros and stores to them are dropped
    auto valid_rows = [&](long long c) -> int {
        const long long rem = t1 - (t0 + c * C);
        return (c < 0 || rem <= 0) ? 0 : (rem < C ? (int)rem : C);
    };
    // first token of chunk c (the sequence start for the placeholder chunks,
    // whose extent is zero)
    auto chunk_tok = [&](long long c) -> long long { return c < 0 ? t0 : t0 + c * C; };
    auto extent = [&](long long c, unsigned row_bytes) -> unsigned {
        const int Cc = valid_rows(c);
        return Cc ? (unsigned)(Cc - 1) * rowb + row_bytes : 0u;
    };
    // A operand of U = T X (or P U): blocks (i, 2kk) and (i, 2kk+1) of a
    // transposed block store; blocks above the diagonal are zero
    auto tile_pair = [&](const bf16 *base, int i, int kk) -> bf16x8 {
        const bf16x4 lo = tile_ld(base + tri(i, 2 * kk) * 256, lane);
        const bf16x4 hi = (2 * kk + 1 <= i) ? tile_ld(base + tri(i, 2 * kk + 1) * 256, lane)
                                            : bf16x4{};
        return cat8(lo, hi);
    };

    if (w < 2) {
        // =================================================================
        // chain waves: value columns 16 ib .. 16 ib + 15 of the slice
        // =================================================================
        const int ib = w;
        f32x4 St[KS];   // S^T[16 Jk + 4 q4 + e][16 ib + l15] (fp32)
#pragma unroll
        for (int jk = 0; jk < KS; ++jk) {
            St[jk] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (a.h0) {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    St[jk][e] = a.h0[sslot + (size_t)(i0 + 16 * ib + l15) * D + 16 * jk + 4 * q4 + e];
            }
        }
        auto publish_state = [&]() {
#pragma unroll
            for (int kk = 0; kk < KD; ++kk) sm.SB[ib][kk][lane] = acc_pair(St[2 * kk], St[2 * kk + 1]);
        };
        publish_state();
        __syncthreads();                      // chunk 0 staged
        __syncthreads();                      // A, P of chunk 0
        __syncthreads();                      // diagonal blocks of T of chunk 0
        int c3 = 0, c2 = 0;   // c mod 3, c mod 2
        for (long long c = 0; c < nch; ++c, c3 = c3 == 2 ? 0 : c3 + 1, c2 ^= 1) {
            const bf16 *Kc = sm.K[c3];
            // ---- alpha: X = V - diag(e^b) K S^T; then the operands of the
            //      state update (k rows are final since their staging), so the
            //      update need not wait on LDS
            f32x4 X[4];
            bf16x8 KT[KS][2];
            f32x4 hs[4];
            float gC;
            {
                const bf16 *Vc = sm.V[c2];
                const float *feb = sm.feb[c3];
                bf16x8 Bs[KD];
#pragma unroll
                for (int kk = 0; kk < KD; ++kk) Bs[kk] = acc_pair(St[2 * kk], St[2 * kk + 1]);
#pragma unroll
                for (int rb = 0; rb < 4; ++rb) {
                    f32x4 xk = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int kk = 0; kk < KD; ++kk)
                        xk = mfma32(frag_rows(Kc, PD, 16 * rb, 32 * kk, lane), Bs[kk], xk);
                    const f32x4 eb = *reinterpret_cast<const f32x4 *>(&feb[16 * rb + 4 * q4]);
                    const bf16x4 vv = frag_col4(Vc, PV, 16 * rb, 16 * ib, lane);
#pragma unroll
                    for (int e = 0; e < 4; ++e) X[rb][e] = (float)vv[e] - eb[e] * xk[e];
                }
                // A operand K^T[16 Jk + l15][s] by transpose loads of the k
                // rows: lane j of each 16-lane group addresses the four stored
                // columns that hold k columns 16 Jk + 4 (j & 3) .. +3
#pragma unroll
                for (int jk = 0; jk < KS; ++jk) {
                    const int pc = 32 * (jk >> 1) + 8 * (l15 & 3) + 4 * (jk & 1);
#pragma unroll
                    for (int kk = 0; kk < 2; ++kk) {
                        const bf16 *p = Kc + (32 * kk + 4 * q4 + (l15 >> 2)) * PD + pc;
                        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(p));
                        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(p + 16 * PD));
                        KT[jk][kk] = cat8(__builtin_bit_cast(bf16x4, lo), __builtin_bit_cast(bf16x4, hi));
                    }
                }
                const float *fhs = sm.fhs[c3];
#pragma unroll
                for (int sb = 0; sb < 4; ++sb) hs[sb] = *reinterpret_cast<const f32x4 *>(&fhs[16 * sb + 4 * q4]);
                gC = sm.fgc[c3][0];
            }
            __syncthreads();
            // ---- beta: U = T X, S^T <- e^{b_C} S^T + K^T diag(e^{b_C - b}) U
            {
                const bf16 *TTc = sm.TT[c2];
                bf16x8 Ta[4][2];
#pragma unroll
                for (int sb = 0; sb < 4; ++sb) {
                    Ta[sb][0] = tile_pair(TTc, sb, 0);
                    Ta[sb][1] = sb >= 2 ? tile_pair(TTc, sb, 1) : bf16x8{};
                }
                const bf16x8 Bx[2] = {acc_pair(X[0], X[1]), acc_pair(X[2], X[3])};
                f32x4 U[4];
#pragma unroll
                for (int sb = 0; sb < 4; ++sb) {
                    U[sb] = mfma32z(Ta[sb][0], Bx[0]);
                    if (sb >= 2) U[sb] = mfma32(Ta[sb][1], Bx[1], U[sb]);
                }
                sm.UB[ib][0][lane] = acc_pair(U[0], U[1]);
                sm.UB[ib][1][lane] = acc_pair(U[2], U[3]);
                f32x4 Uh[4];
#pragma unroll
                for (int sb = 0; sb < 4; ++sb) Uh[sb] = U[sb] * hs[sb];
                const bf16x8 Bh[2] = {acc_pair(Uh[0], Uh[1]), acc_pair(Uh[2], Uh[3])};
#pragma unroll
                for (int jk = 0; jk < KS; ++jk) {
                    f32x4 sv = St[jk] * gC;
                    sv = mfma32(KT[jk][0], Bh[0], sv);
                    sv = mfma32(KT[jk][1], Bh[1], sv);
                    St[jk] = sv;
                }
                publish_state();
            }
            __syncthreads();
        }
        __syncthreads();                      // outputs of the last chunk
        __syncthreads();
        if (a.ht) {
#pragma unroll
            for (int jk = 0; jk < KS; ++jk)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    a.ht[sslot + (size_t)(i0 + 16 * ib + l15) * D + 16 * jk + 4 * q4 + e] = St[jk][e];
        }
        return;
    }

    // =====================================================================
    // waves 2..7
    // =====================================================================
    // ---- staging (waves 4..7): q, k, v of one chunk, a chunk ahead
    const int tl = tid - 256;
    bf16x8 rq[NPC], rk[NPC], rv;
    float rg = 0.f, rbt = 0.f;
#pragma unroll
    for (int i = 0; i < NPC; ++i) rq[i] = rk[i] = bf16x8{};
    rv = bf16x8{};
    // stored chunk m of a row (8 values in paired order) holds columns
    // 32(m>>2) + 4(m&3) .. +3 and the same 16 further on
    auto chunk_col = [](int m) -> int { return 32 * (m >> 2) + 4 * (m & 3); };
    auto stage_load = [&](long long c) {
        const size_t base = (size_t)chunk_tok(c) * tokstride;
        const rsrc_t rqs = make_rsrc(qg + base, extent(c, D * 2));
        const rsrc_t rks = make_rsrc(kg + base, extent(c, D * 2));
#pragma unroll
        for (int i = 0; i < NPC; ++i) {
            const int p = i * 256 + tl;
            const unsigned off = (p / CG) * rowb + 2 * chunk_col(p % CG);
            rq[i] = cat8(bload8(rqs, off), bload8(rqs, off + 32));
            rk[i] = cat8(bload8(rks, off), bload8(rks, off + 32));
        }
        // v slice: 64 rows x 4 pieces of 8 values
        rv = bload16(make_rsrc(vg + base, extent(c, BV * 2)), (tl >> 2) * rowb + 16 * (tl & 3));
        if (w == 4) {   // gate log and beta of row `lane`
            const unsigned hb = (unsigned)(a.H * 4);
            const int Cc = valid_rows(c);
            const unsigned gext = Cc ? (unsigned)(Cc - 1) * hb + 4 : 0u;
            const size_t gbase = (size_t)chunk_tok(c) * a.H + h;
            rg = bload4(make_rsrc(a.g + gbase, gext), lane * hb);
            rbt = bload4(make_rsrc(a.beta + gbase, gext), lane * hb);
        }
    };
    auto stage_store = [&](long long c, int s3) {   // s3 = c mod 3
        bf16 *Qd = sm.Q[c & 1];
        bf16 *Kd = sm.K[s3];
#pragma unroll
        for (int i = 0; i < NPC; ++i) {
            const int p = i * 256 + tl;
            const int o = (p / CG) * PD + 8 * (p % CG);
            *reinterpret_cast<bf16x8 *>(&Qd[o]) = rq[i];
            *reinterpret_cast<bf16x8 *>(&Kd[o]) = rk[i];
        }
        *reinterpret_cast<bf16x8 *>(&sm.V[c & 1][(tl >> 2) * PV + 8 * (tl & 3)]) = rv;
        if (w == 4) {   // inclusive prefix sum of the gate logs over the chunk
            const float b = wave_prefix_sum(rg);
            const float bC = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, b), 63));
            sm.fb[s3][lane] = b;
            sm.feb[s3][lane] = ex(b);
            sm.fhs[s3][lane] = ex(bC - b);
            sm.fbeta[s3][lane] = rbt;
            if (lane == 0) sm.fgc[s3][0] = ex(bC);
        }
    };

    // ---- A, P blocks (waves 2, 3, 6, 7)
    auto frags = [&](const bf16 *M, int blk, bf16x8 (&f)[KD]) {
#pragma unroll
        for (int kk = 0; kk < KD; ++kk) f[kk] = frag_rows(M, PD, 16 * blk, 32 * kk, lane);
    };
    // G = K_J K_I^T and R = K_J Q_I^T: lane holds s = 16J + 4 q4 + e, r = 16I + l15
    auto products = [&](const bf16x8 (&kj)[KD], const bf16x8 (&ki)[KD], const bf16x8 (&qi)[KD],
                        f32x4 &g, f32x4 &p) {
        g = p = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KD; ++kk) {
            g = mfma32(kj[kk], ki[kk], g);
            p = mfma32(kj[kk], qi[kk], p);
        }
    };
    // gate and beta factors of block (I, J): b_r and beta_r of row r = 16I + l15,
    // b_s and beta_s of rows s = 16J + 4 q4 .. +3 (read ahead of the MFMAs)
    struct BlockF { float br, betar; f32x4 bs, betas; };
    auto load_fac = [&](int I, int J, const float *fbv, const float *fbt) -> BlockF {
        BlockF f;
        f.br = fbv[16 * I + l15];
        f.betar = fbt[16 * I + l15];
        f.bs = *reinterpret_cast<const f32x4 *>(&fbv[16 * J + 4 * q4]);
        f.betas = *reinterpret_cast<const f32x4 *>(&fbt[16 * J + 4 * q4]);
        return f;
    };
    // off-diagonal block (I > J): P_IJ^T and L_IJ^T into LDS
    auto put_offdiag = [&](int I, int J, f32x4 g, f32x4 p, const BlockF &F, bf16 *PTn, bf16 *LTn) {
        f32x4 pv, lv;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float f = ex(F.br - F.bs[e]);
            pv[e] = f * p[e];
            lv[e] = F.betar * f * g[e];
        }
        tile_st(PTn + tri(I, J) * 256, lane, pv);
        tile_st(LTn + ltri(I, J) * 256, lane, lv);
    };
    // diagonal block b: P_bb^T into LDS; M = L_bb as acc(M^T), acc(M) (the
    // Gram block is symmetric, so both come from the one product)
    auto diag_prep = [&](int b, f32x4 g, f32x4 p, const BlockF &F, bf16 *PTn, f32x4 &MT, f32x4 &Mn) {
        const int rl = l15;
        f32x4 pv;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int sl = 4 * q4 + e;
            const float d = F.br - F.bs[e];
            const float f = ex(sl <= rl ? d : -d);
            pv[e] = sl <= rl ? f * p[e] : 0.f;
            MT[e] = sl < rl ? F.betar * f * g[e] : 0.f;
            Mn[e] = sl > rl ? F.betas[e] * f * g[e] : 0.f;
        }
        tile_st(PTn + tri(b, b) * 256, lane, pv);
    };
    // Y_bb = (I + M)^{-1} = (I - M)(I + M^2)(I + M^4)(I + M^8) and Y_bb^T; an
    // MFMA with A operand acc(X^T) and B operand acc(Y) yields acc(X Y)
    auto diag_invert = [&](int b, f32x4 MT, f32x4 Mn, f32x4 betas, bf16 *TTn) {
        f32x4 I4;
#pragma unroll
        for (int e = 0; e < 4; ++e) I4[e] = 4 * q4 + e == l15 ? 1.f : 0.f;
        const f32x4 IMn = I4 - Mn, IMT = I4 - MT;
        const f32x4 M2 = mfma16z(cvt4(MT), cvt4(Mn));
        const f32x4 M2T = mfma16z(cvt4(Mn), cvt4(MT));
        const f32x4 Z1 = mfma16(cvt4(M2T), cvt4(IMn), IMn);
        const f32x4 Z1T = mfma16(cvt4(M2), cvt4(IMT), IMT);
        const f32x4 M4 = mfma16z(cvt4(M2T), cvt4(M2));
        const f32x4 M4T = mfma16z(cvt4(M2), cvt4(M2T));
        const f32x4 Z2 = mfma16(cvt4(M4T), cvt4(Z1), Z1);
        const f32x4 Z2T = mfma16(cvt4(M4), cvt4(Z1T), Z1T);
        const f32x4 M8 = mfma16z(cvt4(M4T), cvt4(M4));
        const f32x4 M8T = mfma16z(cvt4(M4), cvt4(M4T));
        const f32x4 Y = mfma16(cvt4(M8T), cvt4(Z2), Z2);
        const f32x4 YT = mfma16(cvt4(M8), cvt4(Z2T), Z2T);
        tile_st(sm.YD[b][0], lane, Y);
        tile_st(sm.YD[b][1], lane, YT);
        tile_st(TTn + tri(b, b) * 256, lane, YT * betas);   // T_bb^T = diag(beta) Y_bb^T
    };
    // ---- outputs (waves 4, 5): O^T = scale (S Q^T diag(e^b) + U^T P^T), so
    //      that a lane ends up with four adjacent columns of one output row;
    //      the published S^T and U operands serve as A operands here and the
    //      q rows and P blocks as B operands
    const int ob = w & 1;          // value block of the output waves
    f32x4 QS[4];                   // (Q S^T)^T[16 ob + 4 q4 + e][16 rb + l15]
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) QS[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
    // one alpha of the output waves: O of chunk c-1 (QS kept from the previous
    // alpha, U and P published since) and QS of chunk c; every LDS operand is
    // read before the first MFMA so the reads overlap
    auto out_step = [&](long long c, int p3, int c3, int cpar) {
        const bf16 *PTp = sm.PT[p3];
        const bf16 *Qc = sm.Q[cpar];
        const bf16x8 Au0 = sm.UB[ob][0][lane], Au1 = sm.UB[ob][1][lane];
        bf16x8 Pb[4][2], As[KD], Qb[4][KD];
        float ebr[4];
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
            Pb[rb][0] = tile_pair(PTp, rb, 0);
            Pb[rb][1] = rb >= 2 ? tile_pair(PTp, rb, 1) : bf16x8{};
            ebr[rb] = sm.feb[c3][16 * rb + l15];
#pragma unroll
            for (int kk = 0; kk < KD; ++kk) Qb[rb][kk] = frag_rows(Qc, PD, 16 * rb, 32 * kk, lane);
        }
#pragma unroll
        for (int kk = 0; kk < KD; ++kk) As[kk] = sm.SB[ob][kk][lane];
        __builtin_amdgcn_sched_barrier(0);
        // O^T of chunk c-1 = QS + U^T P^T, stored as rows
        const rsrc_t ro = make_rsrc(og + (size_t)chunk_tok(c - 1) * tokstride, extent(c - 1, BV * 2));
        const unsigned voff = l15 * rowb + 2 * (16 * ob + 4 * q4);
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
            f32x4 o = mfma32(Au0, Pb[rb][0], QS[rb]);
            if (rb >= 2) o = mfma32(Au1, Pb[rb][1], o);
            bstore8s(ro, voff, 16 * rb * rowb, cvt4(o * a.scale));
        }
        // (diag(e^b) Q S^T)^T of chunk c, S entering chunk c
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
            f32x4 x = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < KD; ++kk) x = mfma32(As[kk], Qb[rb][kk], x);
            QS[rb] = x * ebr[rb];
        }
    };

    // diagonal block of this wave (waves 2, 3, 6, 7), carried from alpha to beta
    const int db = (w & 1) + ((w >> 2) << 1);   // w2 -> 0, w3 -> 1, w6 -> 2, w7 -> 3
    f32x4 dMT = {0.f, 0.f, 0.f, 0.f}, dMn = dMT;

    if (w >= 4) {
        stage_load(0);
        stage_store(0, 0);
        stage_load(1);
        // let the loop be entered with nothing in flight, so the waits inside
        // it follow only the loop's own loads
        __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
    }
    __syncthreads();
    // chunk indices mod 3 and parities of c-1, c, c+1, c+2 (c = -1 first);
    // the output waves and the waves forming T run separate loops with the
    // same barriers, like the chain waves, to keep their registers apart
    int pm3 = 1, cm3 = 2, nm3 = 0, sm3 = 1;
    int cpar = 1;
    auto advance = [&]() {
        pm3 = cm3;
        cm3 = nm3;
        nm3 = sm3;
        sm3 = sm3 == 2 ? 0 : sm3 + 1;
        cpar ^= 1;
    };
    if (w == 4 || w == 5) {
        for (long long c = -1; c <= nch; ++c) {
            out_step(c, pm3, cm3, cpar);
            __syncthreads();
            stage_store(c + 2, sm3);
            stage_load(c + 3);
            __syncthreads();
            advance();
        }
        return;
    }
    for (long long c = -1; c <= nch; ++c) {
        const int npar = cpar ^ 1;
        const bf16 *Kn = sm.K[nm3];
        const bf16 *Qn = sm.Q[npar];
        const float *fbv = sm.fb[nm3];
        const float *fbt = sm.fbeta[nm3];
        bf16 *PTn = sm.PT[nm3];
        // ---------------- alpha: T off the diagonal of chunk c (its diagonal
        // blocks and L came from the previous iteration); diagonal block db of
        // the A and P blocks of chunk c+1.  Every LDS operand first. --------
        BlockF Fd;
        {
            const bf16 *LTc = sm.LT[cpar];
            bf16x4 lt[6], yb[3], ya[3];
#pragma unroll
            for (int t = 0; t < 6; ++t) lt[t] = tile_ld(LTc + t * 256, lane);
#pragma unroll
            for (int t = 0; t < 3; ++t) {
                yb[t] = tile_ld(sm.YD[t][0], lane);        // B operand Y_tt
                ya[t] = tile_ld(sm.YD[t + 1][1], lane);    // acc(Y^T): A operand Y_{t+1,t+1}
            }
            bf16x8 kd[KD], qd[KD];
            frags(Kn, db, kd);
            frags(Qn, db, qd);
            Fd = load_fac(db, db, fbv, fbt);
            // beta_j of the off-diagonal blocks this wave forms: j = 0 (w2),
            // 1 (w3), 2 (w6)
            const float bj = sm.fbeta[cm3][16 * (w == 2 ? 0 : (w == 3 ? 1 : 2)) + l15];
            __builtin_amdgcn_sched_barrier(0);
            if (c >= 0 && w != 7) {
                // Y_ij = -Y_ii sum_k L_ik Y_kj; T_ij = Y_ij diag(beta_j) stored as
                // T_ij^T in accumulator order: element (4 q4 + e, l15) of Y_ij
                // goes to lane 16 (l15 >> 2) + 4 q4 + e
                bf16 *TTc = sm.TT[cpar];
                auto fin = [&](int i, f32x4 v) -> f32x4 { return -mfma16z(ya[i - 1], cvt4(v)); };
                auto putT = [&](int i, int j, f32x4 y) {
                    bf16 *t = TTc + tri(i, j) * 256;
                    const int dl = 16 * (l15 >> 2) + 4 * q4;
#pragma unroll
                    for (int e = 0; e < 4; ++e) t[4 * (dl + e) + (l15 & 3)] = (bf16)(y[e] * bj);
                };
                // L_ij^T blocks: (1,0) 0, (2,0) 1, (2,1) 2, (3,0) 3, (3,1) 4, (3,2) 5
                if (w == 2) {
                    const f32x4 y10 = fin(1, mfma16z(lt[0], yb[0]));
                    const f32x4 y20 = fin(2, mfma16(lt[2], cvt4(y10), mfma16z(lt[1], yb[0])));
                    const f32x4 y30 = fin(3, mfma16(lt[5], cvt4(y20),
                                                    mfma16(lt[4], cvt4(y10), mfma16z(lt[3], yb[0]))));
                    putT(1, 0, y10);
                    putT(2, 0, y20);
                    putT(3, 0, y30);
                } else if (w == 3) {
                    const f32x4 y21 = fin(2, mfma16z(lt[2], yb[1]));
                    const f32x4 y31 = fin(3, mfma16(lt[5], cvt4(y21), mfma16z(lt[4], yb[1])));
                    putT(2, 1, y21);
                    putT(3, 1, y31);
                } else {
                    putT(3, 2, fin(3, mfma16z(lt[5], yb[2])));
                }
            }
            f32x4 g, p;
            products(kd, kd, qd, g, p);
            diag_prep(db, g, p, Fd, PTn, dMT, dMn);
        }
        __syncthreads();
        // ---------------- beta: staging (its loads are long done), then the
        // diagonal inverses of chunk c+1 and its off-diagonal A, P blocks:
        // w2: (1,0), (3,0)  w3: (2,1), (3,1)  w6: (2,0)  w7: (3,2) ----------
        if (w >= 6) {
            stage_store(c + 2, sm3);
            stage_load(c + 3);
        }
        {
            bf16 *LTn = sm.LT[npar];
            const int J = db < 2 ? db : (db == 2 ? 0 : 2);   // 0, 1, 0, 2
            const int I0 = db < 2 ? db + 1 : (db == 2 ? 2 : 3);
            bf16x8 kj[KD], ki[KD], qi[KD], k3[KD], q3[KD];
            frags(Kn, J, kj);
            frags(Kn, I0, ki);
            frags(Qn, I0, qi);
            const BlockF F0 = load_fac(I0, J, fbv, fbt);
            BlockF F3 = F0;
            if (db < 2) {
                frags(Kn, 3, k3);
                frags(Qn, 3, q3);
                F3 = load_fac(3, J, fbv, fbt);
            }
            __builtin_amdgcn_sched_barrier(0);
            diag_invert(db, dMT, dMn, Fd.betas, sm.TT[npar]);
            f32x4 g, p;
            products(kj, ki, qi, g, p);
            put_offdiag(I0, J, g, p, F0, PTn, LTn);
            if (db < 2) {
                products(kj, k3, q3, g, p);
                put_offdiag(3, J, g, p, F3, PTn, LTn);
            }
        }
        __syncthreads();
        advance();
    }
}

}  // namespace

hipError_t launch_prefill_chain(int D, const PrefillArgs &a, hipStream_t s) {
    const long long units = (long long)a.N * a.H;
    if (units <= 0) return hipSuccess;
    const int ntile = D / BV;
    const long long blocks = ((units + 7) / 8) * 8 * ntile;
    dim3 grid((unsigned)blocks), block(NT);
    if (D == 128) hipLaunchKernelGGL((chain_kernel<128>), grid, block, 0, s, a);
    else          hipLaunchKernelGGL((chain_kernel<64>), grid, block, 0, s, a);
    return hipGetLastError();
}

}  // namespace gdr
