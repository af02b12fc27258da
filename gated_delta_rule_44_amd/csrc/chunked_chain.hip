// chunked_chain.hip -- chunked prefill of the gated delta rule for the scalar
// gate (Gated DeltaNet) in two kernels: the chunk-local inverse of every
// chunk in parallel, then the recurrence over chunks with the state on
// dedicated waves.
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
// prep_kernel (one workgroup per chunk and head) forms T, which does not
// depend on the state, and writes it with the chunk's decay factors to a
// record in the workspace, laid out as the MFMA A operands of U = T X (one
// 16-byte piece per lane and operand).  Each diagonal block
// Y_bb = (I + L_bb)^{-1} is the finite series (I - M)(I + M^2)(I + M^4)(I + M^8)
// of its strictly lower 16x16 block M (M^16 = 0), on 16x16x16 MFMAs computed
// in both orientations because an MFMA takes its A operand transposed
// relative to the accumulator layout.  Off the diagonal, block forward
// substitution Y_ij = -Y_ii sum_{k=j}^{i-1} L_ik Y_kj; T = Y diag(beta).
//
// chain_kernel (one workgroup per sequence, head and 32-wide slice of Dv)
// walks the chunks in order.  The only dependency from chunk to chunk is the
// state, through X, U and the update.  Two "chain" waves (SIMDs 0 and 1)
// each own 16 of the 32 value columns and keep their slice of S^T (Dk x 16,
// fp32) in accumulator registers for the whole sequence; they do nothing but
// X, U and the update, and publish S^T and U as bf16 MFMA operands.  Four
// output waves (SIMDs 2 and 3) each own a 16-row block: they load their q
// rows from global memory straight into registers and form P and O one
// chunk behind.  Two staging waves (SIMDs 0 and 1, no MFMA work) bring the
// k rows, the v slice and the chunk's record (T and the decay factors)
// of chunk c+2 into LDS while chunk c runs, their global loads issued one
// and a half iterations before the LDS stores.
// Two barriers per chunk; iteration c:
//   alpha: chain: X, U, state update (chunk c), from registers | output
//          waves: O (c-1) | staging: chunk c+2 from registers into LDS
//   beta:  chain: publish U, S^T; LDS operands of chunk c+1 into registers |
//          output waves: diag(e^b) Q S^T and P (c), global loads of the q
//          rows of c+2 | staging: global loads of chunk c+4
#include "gdr_internal.h"
#include "device_util.h"

namespace gdr {
namespace {

constexpr int C = 64;        // chunk length
constexpr int BV = 32;       // value columns per recurrence workgroup

__device__ inline int tri(int i, int j) { return i * (i + 1) / 2 + j; }   // block (i >= j)
__device__ inline int ltri(int i, int j) { return i * (i - 1) / 2 + j; }  // block (i > j)

// ===========================================================================
// prep_kernel: T of one (chunk, head)
// ===========================================================================
template <int D> struct PrepSmem {
    static constexpr int PD = D + 16;   // conflict-free 16-byte row fragments
    alignas(16) bf16 K[C * PD];
    alignas(16) bf16 TT[10 * 256];      // T_ij^T, i >= j
    alignas(16) bf16 LT[6 * 256];       // L_ij^T, i > j
    alignas(16) bf16 YD[4][2][256];     // Y_bb, Y_bb^T
    alignas(16) float fb[C];            // b_r
    alignas(16) float fbeta[C];         // beta_r
    alignas(16) float frk[C];           // 1 / |k_r| (fused preprocessing)
};

// RAW (fused preprocessing): gate and beta from their logits, the Gram
// blocks scaled by the inverse key norms 1/|k_r| 1/|k_s|, and a 6 KiB
// record whose factor rows are e^{b_r}, e^{b_C - b_r}/|k_r|, e^{b_r}/|k_r|
// and e^{-b_r}/|k_r| (the chain kernel applies 1/|q_r| itself).
template <int D, bool RAW>
__global__ __launch_bounds__(256) void prep_kernel(PrefillArgs a) {
    using Sm = PrepSmem<D>;
    constexpr int PD = Sm::PD;
    constexpr int KD = D / 32;
    constexpr int CG = D / 8;           // 16-byte pieces per row
    constexpr int NPC = C * CG / 256;
    static_assert(NPC >= 1 && (C * CG) % 256 == 0, "staging layout");
    static_assert(kTileBytes == 5 * 1024 + 2 * C * 4, "tile record: T operands, two factor rows");
    constexpr size_t REC = RAW ? kTileBytesRaw : kTileBytes;
    __shared__ Sm sm;

    // ---- which chunk: ci counts chunks over all sequences
    const int h = blockIdx.x % a.H;
    const long long ci = blockIdx.x / a.H;
    long long t0, t1, c;
    if (a.cu_seqlens) {
        if (ci >= a.chunk_base[a.N]) return;
        int lo = 0, hi = a.N - 1;   // the last sequence whose first chunk is <= ci
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (a.chunk_base[mid] <= ci) lo = mid;
            else hi = mid - 1;
        }
        t0 = a.cu_seqlens[lo];
        t1 = a.cu_seqlens[lo + 1];
        c = ci - a.chunk_base[lo];
    } else {
        const long long nch = (a.T + C - 1) / C;
        const long long n = ci / nch;
        c = ci - n * nch;
        t0 = n * a.T;
        t1 = t0 + a.T;
    }
    const long long tc = t0 + c * C;
    const int Cc = (int)(t1 - tc < C ? t1 - tc : C);
    const size_t tokstride = (size_t)a.H * D;
    const unsigned rowb = (unsigned)(tokstride * 2);
    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, l15 = lane & 15, q4 = lane >> 4;

    // ---- k rows (rows past the sequence read as zeros), gate sums
    {
        const size_t base = (size_t)tc * tokstride + (size_t)h * D;
        const rsrc_t rks = make_rsrc(static_cast<const bf16 *>(a.k) + base,
                                     (unsigned)(Cc - 1) * rowb + D * 2);
        bf16x8 vk[NPC];
#pragma unroll
        for (int i = 0; i < NPC; ++i) {
            const int p = i * 256 + tid;
            vk[i] = bload16(rks, (p / CG) * rowb + 16 * (p % CG));
        }
        float gv = 0.f, bv = 0.f;
        if (w == 0) {
            const size_t gb = (size_t)tc * a.H + h;
            if (RAW) {
                // rows past the sequence end keep g = 0 and beta = 0
                const unsigned hx = (unsigned)(a.H * 2);
                const unsigned xext = (unsigned)(Cc - 1) * hx + 2;
                const float xg = bf16_bits_to_float(
                    bload2(make_rsrc(static_cast<const bf16 *>(a.xg) + gb, xext), lane * hx));
                const float xb = bf16_bits_to_float(
                    bload2(make_rsrc(static_cast<const bf16 *>(a.xb) + gb, xext), lane * hx));
                gv = lane < Cc ? neg_softplus(xg, a.gate_scale) : 0.f;
                bv = lane < Cc ? logistic(xb) : 0.f;
            } else {
                const unsigned hb = (unsigned)(a.H * 4);
                const unsigned gext = (unsigned)(Cc - 1) * hb + 4;
                gv = bload4(make_rsrc(a.g + gb, gext), lane * hb);
                bv = bload4(make_rsrc(a.beta + gb, gext), lane * hb);
            }
        }
        if (RAW) {
            // |k_r|^2 over the CG consecutive lanes that hold row r
#pragma unroll
            for (int i = 0; i < NPC; ++i) {
                float ss = 0.f;
#pragma unroll
                for (int u = 0; u < 8; ++u) ss = __builtin_fmaf((float)vk[i][u], (float)vk[i][u], ss);
                ss = sum_group<CG>(ss);
                const int p = i * 256 + tid;
                if (p % CG == 0) sm.frk[p / CG] = inv_norm(ss);
            }
        }
#pragma unroll
        for (int i = 0; i < NPC; ++i) {
            const int p = i * 256 + tid;
            *reinterpret_cast<bf16x8 *>(&sm.K[(p / CG) * PD + 8 * (p % CG)]) = vk[i];
        }
        if (w == 0) {
            sm.fb[lane] = wave_prefix_sum(gv);
            sm.fbeta[lane] = bv;
        }
    }
    __syncthreads();

    auto frags = [&](int blk, bf16x8 (&f)[KD]) {
#pragma unroll
        for (int kk = 0; kk < KD; ++kk) f[kk] = frag_rows(sm.K, PD, 16 * blk, 32 * kk, lane);
    };
    // G = K_J K_I^T: lane holds s = 16J + 4 q4 + e, r = 16I + l15
    auto gram = [&](const bf16x8 (&kj)[KD], const bf16x8 (&ki)[KD]) -> f32x4 {
        f32x4 g = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KD; ++kk) g = mfma32(kj[kk], ki[kk], g);
        return g;
    };
    // Gram block (I, J) of the normalised keys: times 1/|k_r| 1/|k_s|
    auto knorm = [&](int I, int J, f32x4 g) -> f32x4 {
        if (!RAW) return g;
        const float nr = sm.frk[16 * I + l15];
        const f32x4 ns = *reinterpret_cast<const f32x4 *>(&sm.frk[16 * J + 4 * q4]);
        return g * ns * nr;
    };
    // off-diagonal block (I > J) of L, as L_IJ^T
    auto put_L = [&](int I, int J, f32x4 g) {
        const float br = sm.fb[16 * I + l15], betar = sm.fbeta[16 * I + l15];
        const f32x4 bs = *reinterpret_cast<const f32x4 *>(&sm.fb[16 * J + 4 * q4]);
        g = knorm(I, J, g);
        f32x4 lv;
#pragma unroll
        for (int e = 0; e < 4; ++e) lv[e] = betar * ex(br - bs[e]) * g[e];
        tile_st(sm.LT + ltri(I, J) * 256, lane, lv);
    };

    // ---- wave w: diagonal block w of T by the series, and the
    //      off-diagonal blocks of L  w0: (1,0), (3,0)  w1: (2,1), (3,1)
    //      w2: (2,0)  w3: (3,2)
    {
        const int b = w;
        bf16x8 kd[KD];
        frags(b, kd);
        const f32x4 g = knorm(b, b, gram(kd, kd));
        // M = L_bb as acc(M^T) and acc(M): the Gram block is symmetric, so
        // both come from the one product
        const float br = sm.fb[16 * b + l15], betar = sm.fbeta[16 * b + l15];
        const f32x4 bs = *reinterpret_cast<const f32x4 *>(&sm.fb[16 * b + 4 * q4]);
        const f32x4 betas = *reinterpret_cast<const f32x4 *>(&sm.fbeta[16 * b + 4 * q4]);
        f32x4 MT, Mn, I4;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int sl = 4 * q4 + e;
            const float d = br - bs[e];
            const float f = ex(sl <= l15 ? d : -d);
            MT[e] = sl < l15 ? betar * f * g[e] : 0.f;
            Mn[e] = sl > l15 ? betas[e] * f * g[e] : 0.f;
            I4[e] = sl == l15 ? 1.f : 0.f;
        }
        // Y = (I + M)^{-1} = (I - M)(I + M^2)(I + M^4)(I + M^8) and Y^T; an
        // MFMA with A operand acc(X^T) and B operand acc(Y) yields acc(X Y)
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
        tile_st(sm.TT + tri(b, b) * 256, lane, YT * betas);   // T_bb^T = diag(beta) Y_bb^T

        const int J = b < 2 ? b : (b == 2 ? 0 : 2);
        const int I0 = b < 2 ? b + 1 : (b == 2 ? 2 : 3);
        bf16x8 kj[KD], ki[KD];
        frags(J, kj);
        frags(I0, ki);
        put_L(I0, J, gram(kj, ki));
        if (b < 2) {
            frags(3, ki);
            put_L(3, J, gram(kj, ki));
        }
    }
    __syncthreads();

    // ---- T off the diagonal: waves 0, 1, 2 take block columns 0, 1, 2
    if (w < 3) {
        auto LTb = [&](int i, int j) { return tile_ld(sm.LT + ltri(i, j) * 256, lane); };
        auto YB = [&](int j) { return tile_ld(sm.YD[j][0], lane); };   // B operand Y_jj
        auto fin = [&](int i, f32x4 v) -> f32x4 {                      // -Y_ii v
            return -mfma16z(tile_ld(sm.YD[i][1], lane), cvt4(v));
        };
        // T_ij = Y_ij diag(beta_j), stored as T_ij^T in accumulator order:
        // element (4 q4 + e, l15) of Y_ij goes to lane 16 (l15 >> 2) + 4 q4 + e
        const float bj = sm.fbeta[16 * w + l15];
        auto putT = [&](int i, int j, f32x4 y) {
            bf16 *t = sm.TT + tri(i, j) * 256;
            const int dl = 16 * (l15 >> 2) + 4 * q4;
#pragma unroll
            for (int e = 0; e < 4; ++e) t[4 * (dl + e) + (l15 & 3)] = (bf16)(y[e] * bj);
        };
        if (w == 0) {
            const f32x4 y10 = fin(1, mfma16z(LTb(1, 0), YB(0)));
            const f32x4 y20 = fin(2, mfma16(LTb(2, 1), cvt4(y10), mfma16z(LTb(2, 0), YB(0))));
            const f32x4 y30 = fin(3, mfma16(LTb(3, 2), cvt4(y20),
                                            mfma16(LTb(3, 1), cvt4(y10), mfma16z(LTb(3, 0), YB(0)))));
            putT(1, 0, y10);
            putT(2, 0, y20);
            putT(3, 0, y30);
        } else if (w == 1) {
            const f32x4 y21 = fin(2, mfma16z(LTb(2, 1), YB(1)));
            const f32x4 y31 = fin(3, mfma16(LTb(3, 2), cvt4(y21), mfma16z(LTb(3, 1), YB(1))));
            putT(2, 1, y21);
            putT(3, 1, y31);
        } else {
            putT(3, 2, fin(3, mfma16z(LTb(3, 2), YB(2))));
        }
    }
    __syncthreads();

    // ---- the chunk's record in the workspace.  T as MFMA A operands of
    //      U = T X: for row block sb and token blocks (2kk, 2kk+1), lane l
    //      reads its values of the two 16x16 blocks (sb, 2kk), (sb, 2kk+1) as
    //      one 16-byte piece.  The four pairs (1,0), (2,0), (3,0), (3,1) are
    //      stored whole (1 KB each); the pairs (0,0) and (2,1), whose second
    //      block lies above the diagonal, as their first block only (512
    //      bytes).  Then two rows of 64 fp32 decay factors from b_r, the
    //      in-chunk inclusive prefix sums of the gate logs: e^{b_r} and
    //      e^{b_C - b_r}.
    {
        const size_t rec = (size_t)(ci * a.H + h) * REC;
        char *dst = static_cast<char *>(a.tiles) + rec;
        for (int i = tid; i < 4 * 64; i += 256) {
            const int pr = i >> 6, l = i & 63;          // pairs (1,0) (2,0) (3,0) (3,1)
            const int sb = pr == 0 ? 1 : (pr == 1 ? 2 : 3);
            const int kk = pr == 3 ? 1 : 0;
            reinterpret_cast<bf16x8 *>(dst)[i] = cat8(tile_ld(sm.TT + tri(sb, 2 * kk) * 256, l),
                                                      tile_ld(sm.TT + tri(sb, 2 * kk + 1) * 256, l));
        }
        if (tid < 2 * 64) {                             // first blocks of (0,0), (2,1)
            const int l = tid & 63;
            reinterpret_cast<bf16x4 *>(dst + 4096)[tid] = tile_ld(sm.TT + (tid < 64 ? tri(0, 0) : tri(2, 2)) * 256, l);
        } else if (tid < 2 * 64 + C) {
            const int r = tid - 2 * 64;
            float *f = reinterpret_cast<float *>(dst + 5120);
            const float b = sm.fb[r];
            f[r] = ex(b);
            if (RAW) {
                const float nk = sm.frk[r];
                f[C + r] = ex(sm.fb[C - 1] - b) * nk;
                f[2 * C + r] = ex(b) * nk;
                f[3 * C + r] = ex(-b) * nk;
            } else {
                f[C + r] = ex(sm.fb[C - 1] - b);
            }
        }
    }
}

// ===========================================================================
// chain_kernel: the recurrence over chunks
// ===========================================================================
// the chunk's workspace record as the prep kernel writes it
template <bool RAW> struct TRecT {
    bf16x8 pairs[4][64];            // T operand pairs (1,0), (2,0), (3,0), (3,1)
    bf16x4 halves[2][64];           // first blocks of the pairs (0,0), (2,1)
    float eb[C];                    // e^{b_r}
    float hs[C];                    // e^{b_C - b_r}
};
template <> struct TRecT<true> {
    bf16x8 pairs[4][64];
    bf16x4 halves[2][64];
    float eb[C];                    // e^{b_r}
    float hs[C];                    // e^{b_C - b_r} / |k_r|
    float ek[C];                    // e^{b_r} / |k_r|
    float nk[C];                    // e^{-b_r} / |k_r|
};

template <int D, bool RAW> struct ChainSmem {
    // k rows; a row stride of 8 x odd dwords keeps the 16-byte row fragment
    // reads free of bank conflicts (and halves those of the transpose reads,
    // against 4 x odd)
    static constexpr int PD = D + 16;
    static constexpr int KD = D / 32;
    // v slice rows [r][i]; a stride of 24 dwords puts the 8 rows that one
    // transpose load touches per half-wave on disjoint banks
    static constexpr int PV = BV + 16;
    using TRec = TRecT<RAW>;
    alignas(16) bf16 K[3][C * PD];      // by chunk mod 3
    alignas(16) bf16 V[3][C * PV];      // by chunk mod 3
    alignas(16) TRec TR[3];             // by chunk mod 3
    alignas(16) bf16x8 SB[2][2][KD][64];// S^T entering a chunk (by parity), per chain wave
    alignas(16) bf16x8 UB[2][2][64];    // U as operands, per chain wave
};

template <int D, bool RAW>
__global__ __launch_bounds__(512, 1) void chain_kernel(PrefillArgs a) {
    using Sm = ChainSmem<D, RAW>;
    constexpr size_t REC = RAW ? kTileBytesRaw : kTileBytes;
    constexpr int PD = Sm::PD;
    constexpr int PV = Sm::PV;
    constexpr int NTILE = D / BV;
    constexpr int KD = Sm::KD;          // 32-wide k steps over Dk
    constexpr int KS = D / 16;          // 16-row blocks of S^T
    constexpr int CG = D / 8;           // 16-byte pieces per k row
    // staged pieces (16 bytes) per chunk: k rows, v slice rows, T record
    constexpr int NKP = C * CG, NVP = C * BV / 8, NTP = (int)(REC / 16);
    constexpr int NST = NKP + NVP + NTP;
    constexpr int NI = (NST + 127) / 128;   // per staging thread
    static_assert(NKP % 64 == 0 && NVP % 64 == 0, "staging layout");
    static_assert(sizeof(typename Sm::TRec) == REC, "tile record layout");
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
    long long t0, t1, cbase;
    if (a.cu_seqlens) {
        t0 = a.cu_seqlens[n];
        t1 = a.cu_seqlens[n + 1];
        cbase = a.chunk_base[n];
    } else {
        t0 = (long long)n * a.T;
        t1 = t0 + a.T;
        cbase = (long long)n * ((a.T + C - 1) / C);
    }
    const int i0 = tile * BV;
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

    // rows of chunk c that exist (0 past the end and for c < 0); buffer
    // extents cover just these, so loads of other rows return zeros and
    // stores to them are dropped
    auto valid_rows = [&](long long c) -> int {
        const long long rem = t1 - (t0 + c * C);
        return (c < 0 || rem <= 0) ? 0 : (rem < C ? (int)rem : C);
    };
    // first token of chunk c (the sequence start for c < 0, whose extent is 0)
    auto chunk_tok = [&](long long c) -> long long { return c < 0 ? t0 : t0 + c * C; };
    auto extent = [&](long long c, unsigned row_bytes) -> unsigned {
        const int Cc = valid_rows(c);
        return Cc ? (unsigned)(Cc - 1) * rowb + row_bytes : 0u;
    };
    // The k index of the state.  A 16x16x32 MFMA sums over k; lane l of a
    // row-fragment operand (16 bytes of one k row) supplies k = 32 kk + 8 (l >> 4)
    // + u, u = 0..7.  The S^T accumulator blocks are numbered so that the pair
    // (2 kk, 2 kk + 1) supplies exactly these k as the other operand: block jk
    // holds rows 32 (jk >> 1) + 8 q4 + 4 (jk & 1) + e of S^T in lane (q4, e).
    auto srow = [&](int jk, int e) -> int { return 32 * (jk >> 1) + 8 * q4 + 4 * (jk & 1) + e; };
    const std::integral_constant<int, 0> R0;
    const std::integral_constant<int, 1> R1;

    if (w < 2) {
        // =================================================================
        // chain waves: value columns 16 ib .. 16 ib + 15 of the slice
        // =================================================================
        const int ib = w;
        // S^T[srow(jk, e)][16 ib + l15] (fp32); the four rows e of a block are
        // adjacent columns of S, so they move as one 16-byte access
        f32x4 St[KS];
        const size_t srow0 = (size_t)(i0 + 16 * ib + l15) * D;
        const float *h0p = seq_h0<D>(a, n, h);
#pragma unroll
        for (int jk = 0; jk < KS; ++jk)
            St[jk] = h0p ? *reinterpret_cast<const f32x4 *>(h0p + srow0 + srow(jk, 0))
                         : f32x4{0.f, 0.f, 0.f, 0.f};
        auto publish_state = [&](int spar) {   // S^T entering a chunk of parity spar
#pragma unroll
            for (int kk = 0; kk < KD; ++kk) sm.SB[spar][ib][kk][lane] = acc_pair(St[2 * kk], St[2 * kk + 1]);
        };
        // operands of a chunk, read a phase ahead of their use: k row
        // fragments, K^T, the v slice, T and the decay factors.  K^T comes
        // from transpose loads of the k rows: lane j of each 16-lane group
        // addresses k columns 32 (jk >> 1) + 8 (j & 3) + 4 (jk & 1) .. +3, so
        // output lane i receives k = srow(jk, .) for row i of the block.
        bf16x8 Kf[4][KD], KT[KS][2], Ta[4][2];
        bf16x4 vv[4];
        f32x4 eb[4], hs[4];
        float gC = 0.f;
        auto prefetch = [&](long long c, int m3) {
            const bf16 *Kc = sm.K[m3];
            const bf16 *Vc = sm.V[m3];
            const typename Sm::TRec &R = sm.TR[m3];
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
#pragma unroll
            for (int rb = 0; rb < 4; ++rb) {
#pragma unroll
                for (int kk = 0; kk < KD; ++kk) Kf[rb][kk] = frag_rows(Kc, PD, 16 * rb, 32 * kk, lane);
                vv[rb] = frag_col4(Vc, PV, 16 * rb, 16 * ib, lane);
                if constexpr (RAW) eb[rb] = *reinterpret_cast<const f32x4 *>(&R.ek[16 * rb + 4 * q4]);
                else               eb[rb] = *reinterpret_cast<const f32x4 *>(&R.eb[16 * rb + 4 * q4]);
                hs[rb] = *reinterpret_cast<const f32x4 *>(&R.hs[16 * rb + 4 * q4]);
                Ta[rb][0] = rb == 0 ? cat8(R.halves[0][lane], bf16x4{}) : R.pairs[rb - 1][lane];
                Ta[rb][1] = rb == 2 ? cat8(R.halves[1][lane], bf16x4{})
                          : (rb == 3 ? R.pairs[3][lane] : bf16x8{});
            }
            gC = R.eb[C - 1];
        };
        publish_state(0);
        __syncthreads();                      // chunks 0 and 1 staged
        prefetch(0, 0);
        int m3 = 0;                           // c mod 3
        for (long long c = 0; c < nch; ++c) {
            const int par = (int)(c & 1);
            const int n3 = m3 == 2 ? 0 : m3 + 1;
            if (a.states) {                   // the state entering chunk c
                float *sp = a.states + ((size_t)(cbase + c) * a.H + h) * D * D + srow0;
#pragma unroll
                for (int jk = 0; jk < KS; ++jk) *reinterpret_cast<f32x4 *>(sp + srow(jk, 0)) = St[jk];
            }
            // ---- alpha: X = V - diag(e^b) K S^T, U = T X and the state
            //      update, all from registers
            f32x4 X[4];
            {
                bf16x8 Bs[KD];
#pragma unroll
                for (int kk = 0; kk < KD; ++kk) Bs[kk] = acc_pair(St[2 * kk], St[2 * kk + 1]);
                f32x4 xk[4];
#pragma unroll
                for (int rb = 0; rb < 4; ++rb) {
                    xk[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int kk = 0; kk < KD; ++kk) xk[rb] = mfma32(Kf[rb][kk], Bs[kk], xk[rb]);
                }
#pragma unroll
                for (int rb = 0; rb < 4; ++rb)
#pragma unroll
                    for (int e = 0; e < 4; ++e) X[rb][e] = (float)vv[rb][e] - eb[rb][e] * xk[rb][e];
            }
            // U = T X, S^T <- e^{b_C} S^T + K^T diag(e^{b_C - b}) U
            bf16x8 Ub[2];
            {
                const bf16x8 Bx[2] = {acc_pair(X[0], X[1]), acc_pair(X[2], X[3])};
                f32x4 U[4];
#pragma unroll
                for (int sb = 0; sb < 4; ++sb) {
                    U[sb] = mfma32z(Ta[sb][0], Bx[0]);
                    if (sb >= 2) U[sb] = mfma32(Ta[sb][1], Bx[1], U[sb]);
                }
                Ub[0] = acc_pair(U[0], U[1]);
                Ub[1] = acc_pair(U[2], U[3]);
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
            }
            __syncthreads();
            // ---- beta: publish U and S^T; operands of the next chunk
            sm.UB[ib][0][lane] = Ub[0];
            sm.UB[ib][1][lane] = Ub[1];
            publish_state(par ^ 1);
            prefetch(c + 1, n3);
            __syncthreads();
            m3 = n3;
        }
        __syncthreads();                      // outputs of the last chunk
        __syncthreads();
        if (float *htp = seq_ht<D>(a, n, h)) {
#pragma unroll
            for (int jk = 0; jk < KS; ++jk) *reinterpret_cast<f32x4 *>(htp + srow0 + srow(jk, 0)) = St[jk];
        }
        return;
    }

    if (w >= 4 && w < 6) {
        // =================================================================
        // staging waves: k rows, the v slice and the record (T, factors) of
        // chunk c+2 into LDS during alpha of iteration c, from registers
        // loaded during beta of iteration c-2 (two register sets)
        // =================================================================
        const int tl = tid - 256;
        bf16x8 rs[2][NI];
        auto st_load = [&](long long c, auto S) {
            constexpr int r = decltype(S)::value;
            const size_t base = (size_t)chunk_tok(c) * tokstride;
            const rsrc_t rks = make_rsrc(kg + base, extent(c, D * 2));
            const rsrc_t rvs = make_rsrc(vg + base, extent(c, BV * 2));
            const bool have = valid_rows(c) > 0 && cbase + c < a.max_chunks;
            const size_t rec = (size_t)((have ? cbase + c : 0) * a.H + h) * REC;
            const rsrc_t rts = make_rsrc(static_cast<const char *>(a.tiles) + rec,
                                         have ? (unsigned)REC : 0u);
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                const int p0 = i * 128 + 64 * (w - 4);   // this wave's first piece
                const int p = i * 128 + tl;
                if (p0 < NKP) {
                    rs[r][i] = bload16(rks, (p / CG) * rowb + 16 * (p % CG));
                } else if (p0 < NKP + NVP) {
                    const int pv = p - NKP;
                    rs[r][i] = bload16(rvs, (pv >> 2) * rowb + 16 * (pv & 3));
                } else {
                    rs[r][i] = bload16(rts, 16 * (p - NKP - NVP));
                }
            }
        };
        auto st_store = [&](int m3, auto S) {   // chunk c into slot m3 = c mod 3
            constexpr int r = decltype(S)::value;
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                const int p0 = i * 128 + 64 * (w - 4);
                const int p = i * 128 + tl;
                if (p0 < NKP) {
                    *reinterpret_cast<bf16x8 *>(&sm.K[m3][(p / CG) * PD + 8 * (p % CG)]) = rs[r][i];
                } else if (p0 < NKP + NVP) {
                    const int pv = p - NKP;
                    *reinterpret_cast<bf16x8 *>(&sm.V[m3][(pv >> 2) * PV + 8 * (pv & 3)]) = rs[r][i];
                } else if (p < NST) {
                    reinterpret_cast<bf16x8 *>(&sm.TR[m3])[p - NKP - NVP] = rs[r][i];
                }
            }
        };
        st_load(0, R0);
        st_store(0, R0);
        st_load(1, R0);
        st_store(1, R0);
        st_load(2, R0);
        st_load(3, R1);
        __syncthreads();
        int m3 = 2;                           // (c + 2) mod 3
        for (long long c = 0;; c += 2) {
            st_store(m3, R0);
            m3 = m3 == 2 ? 0 : m3 + 1;
            __syncthreads();
            st_load(c + 4, R0);
            __syncthreads();
            if (c + 1 > nch) break;
            st_store(m3, R1);
            m3 = m3 == 2 ? 0 : m3 + 1;
            __syncthreads();
            st_load(c + 5, R1);
            __syncthreads();
            if (c + 2 > nch) break;
        }
        return;
    }

    // =====================================================================
    // output waves: row block RB of the chunk (waves 2, 3, 7, 6 take 0, 1, 2,
    // 3, so each of SIMDs 2 and 3 carries 1 + 4 or 2 + 3 blocks of P), both
    // value blocks.  O^T = scale (S Q^T diag(e^b) + U^T P^T) so that a lane
    // ends up with four adjacent columns of one output row: the published
    // S^T and U serve as A operands, the q rows and P^T as B operands.  P^T
    // is formed in accumulator registers, so it feeds the MFMA directly.
    // Iteration c, alpha: O of chunk c-1 (U of chunk c-1 was published during
    // beta of c-1); beta: QS and P of chunk c (S^T entering chunk c was
    // published during beta of c-1, and chunk c's k rows stay in LDS until
    // alpha of c+1), then the q rows of chunk c+2, from global memory
    // straight into registers.
    // =====================================================================
    auto out_loop = [&](auto RBc) {
        constexpr int RB = decltype(RBc)::value;
        constexpr int NP2 = (RB + 2) / 2;   // pairs of 16-token blocks J <= RB
        bf16x8 Qr[2][KD];                   // q rows 16 RB + l15, two chunks
        bf16x8 Pp[NP2];                     // P^T of the previous chunk, as B operand pairs
        f32x4 QSp[2];                       // (Q S^T)^T[16 ob + 4 q4 + e][16 RB + l15], scaled by e^b
        auto q_load = [&](long long c, auto S) {
            constexpr int r = decltype(S)::value;
            const rsrc_t rq = make_rsrc(qg + (size_t)chunk_tok(c) * tokstride, extent(c, D * 2));
            const unsigned off = (16 * RB + l15) * rowb + 16 * q4;
#pragma unroll
            for (int kk = 0; kk < KD; ++kk) Qr[r][kk] = bload16(rq, off + 64 * kk);
        };
        // O of chunk c-1
        auto o_step = [&](long long c) {
            bf16x8 Au[2][NP2];
#pragma unroll
            for (int ob = 0; ob < 2; ++ob)
#pragma unroll
                for (int k2 = 0; k2 < NP2; ++k2) Au[ob][k2] = sm.UB[ob][k2][lane];
            const rsrc_t ro = make_rsrc(og + (size_t)chunk_tok(c - 1) * tokstride, extent(c - 1, BV * 2));
            const unsigned voff = l15 * rowb + 8 * q4;
#pragma unroll
            for (int ob = 0; ob < 2; ++ob) {
                f32x4 o = QSp[ob];
#pragma unroll
                for (int k2 = 0; k2 < NP2; ++k2) o = mfma32(Au[ob][k2], Pp[k2], o);
                bstore8s(ro, voff + 32 * ob, 16 * RB * rowb, cvt4(o * a.scale));
            }
        };
        // QS and P of chunk c (m3 = c mod 3)
        auto qp_step = [&](long long c, int m3, auto S) {
            constexpr int r = decltype(S)::value;
            const bf16 *Kc = sm.K[m3];
            bf16x8 As[2][KD], Kj[RB + 1][KD];
            f32x4 nebJ[RB + 1];
#pragma unroll
            for (int ob = 0; ob < 2; ++ob)
#pragma unroll
                for (int kk = 0; kk < KD; ++kk) As[ob][kk] = sm.SB[(int)(c & 1)][ob][kk][lane];
#pragma unroll
            for (int J = 0; J <= RB; ++J) {
#pragma unroll
                for (int kk = 0; kk < KD; ++kk) Kj[J][kk] = frag_rows(Kc, PD, 16 * J, 32 * kk, lane);
                if constexpr (RAW) {
                    nebJ[J] = *reinterpret_cast<const f32x4 *>(&sm.TR[m3].nk[16 * J + 4 * q4]);
                } else {
                    const f32x4 ebJ = *reinterpret_cast<const f32x4 *>(&sm.TR[m3].eb[16 * J + 4 * q4]);
#pragma unroll
                    for (int e = 0; e < 4; ++e) nebJ[J][e] = __builtin_amdgcn_rcpf(ebJ[e]);   // e^{-b_s}
                }
            }
            float ebr = sm.TR[m3].eb[16 * RB + l15];
            if constexpr (RAW) {
                // 1/|q_r| for the lane's row: its 8 KD values, then the four
                // lanes (q4) that share the row
                float ss = 0.f;
#pragma unroll
                for (int kk = 0; kk < KD; ++kk)
#pragma unroll
                    for (int u = 0; u < 8; ++u) ss = __builtin_fmaf((float)Qr[r][kk][u], (float)Qr[r][kk][u], ss);
                ss = swap_sum32(swap_sum16(ss));
                ebr *= inv_norm(ss);
            }
            // diag(e^b) Q S^T (S entering chunk c)
#pragma unroll
            for (int ob = 0; ob < 2; ++ob) {
                f32x4 x = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < KD; ++kk) x = mfma32(As[ob][kk], Qr[r][kk], x);
                QSp[ob] = x * ebr;
            }
            // P: K_J Q_RB^T gives lane s = 16 J + 4 q4 + e, r = 16 RB + l15,
            // and P[r][s] = e^{b_r} e^{-b_s} q_r.k_s for s <= r
            f32x4 pv[RB + 2];
#pragma unroll
            for (int J = 0; J <= RB; ++J) {
                f32x4 p = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < KD; ++kk) p = mfma32(Kj[J][kk], Qr[r][kk], p);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float v = ebr * nebJ[J][e] * p[e];
                    pv[J][e] = (J < RB || 4 * q4 + e <= l15) ? v : 0.f;
                }
            }
            pv[RB + 1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int k2 = 0; k2 < NP2; ++k2) Pp[k2] = acc_pair(pv[2 * k2], pv[2 * k2 + 1]);
        };
        q_load(0, R0);
        q_load(1, R1);
        QSp[0] = QSp[1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k2 = 0; k2 < NP2; ++k2) Pp[k2] = bf16x8{};
        __syncthreads();
        int m3 = 0;                           // c mod 3
        for (long long c = 0;; c += 2) {
            o_step(c);
            __syncthreads();
            qp_step(c, m3, R0);
            q_load(c + 2, R0);
            m3 = m3 == 2 ? 0 : m3 + 1;
            __syncthreads();
            if (c + 1 > nch) break;
            o_step(c + 1);
            __syncthreads();
            qp_step(c + 1, m3, R1);
            q_load(c + 3, R1);
            m3 = m3 == 2 ? 0 : m3 + 1;
            __syncthreads();
            if (c + 2 > nch) break;
        }
    };
    if (w == 2)      out_loop(std::integral_constant<int, 0>{});
    else if (w == 3) out_loop(std::integral_constant<int, 1>{});
    else if (w == 7) out_loop(std::integral_constant<int, 2>{});
    else             out_loop(std::integral_constant<int, 3>{});
}

// First chunk of every packed sequence: base[n] = sum over m < n of
// ceil(len_m / C), base[N] = the total.  One workgroup: each thread sums a
// run of consecutive sequences, then an exclusive scan over the 256 runs.
__global__ __launch_bounds__(256) void chunk_base_kernel(const int32_t *cu, int N, int32_t *base) {
    __shared__ int part[256];
    const int t = threadIdx.x;
    const int per = (N + 255) / 256;
    const int m0 = t * per < N ? t * per : N;
    const int m1 = m0 + per < N ? m0 + per : N;
    int s = 0;
    for (int m = m0; m < m1; ++m) s += (cu[m + 1] - cu[m] + C - 1) / C;
    part[t] = s;
    __syncthreads();
    for (int d = 1; d < 256; d <<= 1) {   // inclusive scan (Hillis-Steele)
        const int x = t >= d ? part[t - d] : 0;
        __syncthreads();
        part[t] += x;
        __syncthreads();
    }
    int acc = part[t] - s;                // exclusive
    for (int m = m0; m < m1; ++m) {
        base[m] = acc;
        acc += (cu[m + 1] - cu[m] + C - 1) / C;
    }
    if (t == 255) base[N] = part[255];
}

}  // namespace

hipError_t launch_chunk_base(const int32_t *cu_seqlens, int N, int32_t *chunk_base,
                             hipStream_t s) {
    if (N < 0) return hipErrorInvalidValue;
    hipLaunchKernelGGL(chunk_base_kernel, dim3(1), dim3(256), 0, s, cu_seqlens, N, chunk_base);
    return hipGetLastError();
}

hipError_t launch_prefill_chain(int D, const PrefillArgs &a, hipStream_t s) {
    const long long units = (long long)a.N * a.H;
    if (units <= 0) return hipSuccess;
    if (a.cu_seqlens) {
        hipLaunchKernelGGL(chunk_base_kernel, dim3(1), dim3(256), 0, s, a.cu_seqlens, a.N,
                           a.chunk_base);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const long long prep_blocks = a.max_chunks * a.H;
    if (prep_blocks > 0) {
        dim3 grid((unsigned)prep_blocks), block(256);
        if (a.xg) {
            if (D == 128) hipLaunchKernelGGL((prep_kernel<128, true>), grid, block, 0, s, a);
            else          hipLaunchKernelGGL((prep_kernel<64, true>), grid, block, 0, s, a);
        } else {
            if (D == 128) hipLaunchKernelGGL((prep_kernel<128, false>), grid, block, 0, s, a);
            else          hipLaunchKernelGGL((prep_kernel<64, false>), grid, block, 0, s, a);
        }
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const int ntile = D / BV;
    const long long blocks = ((units + 7) / 8) * 8 * ntile;
    dim3 grid((unsigned)blocks), block(512);
    if (a.xg) {
        if (D == 128) hipLaunchKernelGGL((chain_kernel<128, true>), grid, block, 0, s, a);
        else          hipLaunchKernelGGL((chain_kernel<64, true>), grid, block, 0, s, a);
    } else {
        if (D == 128) hipLaunchKernelGGL((chain_kernel<128, false>), grid, block, 0, s, a);
        else          hipLaunchKernelGGL((chain_kernel<64, false>), grid, block, 0, s, a);
    }
    return hipGetLastError();
}

}  // namespace gdr
