// fa_bwd.hip -- exact-attention backward with recomputation for gfx950.
//
// The scores are never stored: each workgroup recomputes S = Q K^T and
// P = exp(scale S - LSE) tile by tile from the saved per-row log-sum-exp
// ("Flash Attention uitgelegd", section "Recomputation"; Slovak page,
// section 2).  The gradients are the chain rule through the forward
// definition:
//     dV = P^T dO,  dP = dO V^T,  D_i = sum_k dO_ik O_ik,
//     dS = P * (dP - D),  dK = scale dS^T Q,  dQ = scale dS K.
//
// Three launches on the caller's stream:
//   1. bwd_prep:  D = rowsum(dO * O) in fp32, and the fp32 dQ accumulator
//                 cleared to zero.
//   2. bwd_main:  one workgroup per tile of BC = 128 keys of one head (4 waves,
//                 32 keys each).  K and V of the tile stay in registers (and K
//                 also in LDS); the workgroup walks the query tiles (BR = 64
//                 rows) that can see its keys.  Q, dO, LSE and D of the next
//                 query tile are copied global -> LDS while the current one is
//                 computed.  dK^T and dV^T accumulate in registers; dS goes
//                 through LDS so that all four waves contribute to
//                 dQ_i += dS K_j, which is added into the fp32 accumulator with
//                 global atomics that stay in flight across the barriers.
//   3. bwd_dq:    dQ = scale * accumulator, rounded to bf16.
//
// Layout trick (as in the forward): S is computed with queries as MFMA rows
// and keys as columns, so each lane holds one key and 16 queries; those
// registers are directly the K-slot-ordered B operands of dV^T = dO^T P and
// dK^T = Q^T dS, whose Q^T / dO^T operands are read with the transposing LDS
// read in the matching query order.
#include "fa_common.hpp"
#include "fa_internal.hpp"

namespace fa {

namespace {

constexpr int BWD_BR = 64;       // query rows per inner step
constexpr int BWD_BC = 128;      // keys per workgroup (4 waves x 32)
constexpr int BWD_THREADS = 256;

// ---------------------------------------------------------------------------
// 1. D = rowsum(dO * O); zero the dQ accumulator.  d/8 lanes per row.
// ---------------------------------------------------------------------------
template <int D, bool O_BF16>
__global__ void __launch_bounds__(256)
bwd_prep_kernel(const void* __restrict__ O, const __bf16* __restrict__ dO, float* __restrict__ delta,
                float* __restrict__ dq_acc, long long rows) {
    constexpr int LPR = D / 8;
    const long long gid = (long long)blockIdx.x * 256 + threadIdx.x;
    const long long row = gid / LPR;
    const int part = (int)(gid % LPR);
    const bool live = row < rows;
    float acc = 0.f;
    if (live) {
        const size_t base = (size_t)row * D + 8 * part;
        const uint4 du = *reinterpret_cast<const uint4*>(dO + base);
        const uint32_t* dp = reinterpret_cast<const uint32_t*>(&du);
        float ov[8];
        if (O_BF16) {
            const uint4 ou = *reinterpret_cast<const uint4*>(static_cast<const __bf16*>(O) + base);
            const uint32_t* op = reinterpret_cast<const uint32_t*>(&ou);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                ov[2 * j] = bf16_lo(op[j]);
                ov[2 * j + 1] = bf16_hi(op[j]);
            }
        } else {
            const float4 a = *reinterpret_cast<const float4*>(static_cast<const float*>(O) + base);
            const float4 b = *reinterpret_cast<const float4*>(static_cast<const float*>(O) + base + 4);
            ov[0] = a.x; ov[1] = a.y; ov[2] = a.z; ov[3] = a.w;
            ov[4] = b.x; ov[5] = b.y; ov[6] = b.z; ov[7] = b.w;
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            acc = fmaf(bf16_lo(dp[j]), ov[2 * j], acc);
            acc = fmaf(bf16_hi(dp[j]), ov[2 * j + 1], acc);
        }
        const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
        *reinterpret_cast<float4*>(dq_acc + base) = z;
        *reinterpret_cast<float4*>(dq_acc + base + 4) = z;
    }
    acc = (LPR == 16) ? dpp_sum16(acc) : dpp_sum8(acc);
    if (live && part == 0) delta[row] = acc;
}

// ---------------------------------------------------------------------------
// 2. main kernel
// ---------------------------------------------------------------------------
// Q, dO and K tiles live in LDS row-major (2*D bytes per row, no padding),
// filled by direct global -> LDS copies.  Each is read two ways: 16-byte
// chunks by 32 consecutive rows (A operands of S = Q K^T and dP = dO V^T) and
// with the transposing 8-byte read (Q^T, dO^T and K^T operands, 4 rows x 32
// bytes per 16-lane group).  The XOR of the 16-byte chunk index with
// 4*(row%4) + (row/4)%4 keeps both patterns free of bank conflicts.
template <int D>
__device__ __forceinline__ int bwd_swz(int row) {
    return (4 * (row & 3) + ((row >> 2) & 3)) & (D / 8 - 1);
}

// s_waitcnt with only vmcnt constrained (expcnt / lgkmcnt left at their max).
#define FA_WAIT_VMCNT(n) \
    __builtin_amdgcn_s_waitcnt((((n) & 15) | (((n) >> 4) << 14)) | (7 << 4) | (15 << 8))
#define FA_WAIT_LGKM0() __builtin_amdgcn_s_waitcnt((15) | (3 << 14) | (7 << 4))

template <int D, bool CAUSAL>
__global__ void __launch_bounds__(BWD_THREADS)
bwd_main_kernel(const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
                const __bf16* __restrict__ dO, const float* __restrict__ LSE,
                const float* __restrict__ delta, float* __restrict__ dq_acc, __bf16* __restrict__ dK,
                __bf16* __restrict__ dV, int BH, int N, float c /* scale*log2e */, float scale) {
    constexpr int BR = BWD_BR, BC = BWD_BC;
    constexpr int ROWB = 2 * D;                  // bytes per row of a Q/dO/K tile
    constexpr int CPR = D / 8;
    constexpr int QTB = BR * ROWB;               // bytes of a Q (or dO) tile
    constexpr int KTB = BC * ROWB;               // bytes of the K tile
    constexpr int RPS = 1024 / ROWB;             // rows per 1 KiB copy segment
    constexpr int QSPW = QTB / 1024 / 4;         // Q segments per wave
    constexpr int KSPW = KTB / 1024 / 4;         // K segments per wave
    constexpr int DSS = BC + 8;                  // dS row stride (bf16)
    constexpr int NQB = BR / 32;
    constexpr int DQ_UNITS = NQB * (D / 32);     // 32x32 output blocks of dQ per tile
    constexpr int DQ_PER_WAVE = DQ_UNITS / 4;
    constexpr int ATOMICS = DQ_PER_WAVE * 16;    // VMEM atomics a wave issues per tile
    static_assert(QSPW >= 1 && DQ_UNITS % 4 == 0, "tile shapes");

    // Two buffers, each holding a query tile's Q, dO, LSE and D, plus the K
    // tile and dS.  The buffers are separate LDS objects, so the compiler can
    // tell that the copies into one do not alias the reads of the other and
    // need not wait for them.
    constexpr int BUFB = 2 * QTB + 2 * BR * 4;
    __shared__ __attribute__((aligned(1024))) char buf0[BUFB];
    __shared__ __attribute__((aligned(1024))) char buf1[BUFB];
    __shared__ __attribute__((aligned(1024))) char kbuf[KTB];
    __shared__ __attribute__((aligned(16))) __bf16 dss[BR * DSS];
    static_assert(BR == 64, "one wave copies a row statistic of the tile");

    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const int l32 = lane & 31, g = lane >> 5;

    // heavy tiles first: key tile 0 sees every query tile
    const int bh = blockIdx.x % BH;
    const int kt = blockIdx.x / BH;
    const int k0 = kt * BC;
    const size_t hoff = (size_t)bh * (size_t)N * D;
    const __bf16* Qh = Q + hoff;
    const __bf16* Kh = K + hoff;
    const __bf16* Vh = V + hoff;
    const __bf16* dOh = dO + hoff;
    const float* LSEh = LSE + (size_t)bh * N;
    const float* Dh = delta + (size_t)bh * N;
    float* dQh = dq_acc + hoff;

    // copy rows [r0, r0 + rows) of a [N, D] tensor into an LDS tile
    // (segments seg0 .. seg0+nseg-1); rows past the end are clamped to N-1
    auto issue = [&](const __bf16* src, int r0, char* dst, int seg0, int nseg) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < nseg; ++i) {
            const int seg = seg0 + i;
            const int row = seg * RPS + lane / CPR;
            const int pc = lane % CPR;
            const size_t grow = (size_t)min(r0 + row, N - 1) * D;
            g2lds16(src + grow + 8 * (pc ^ bwd_swz<D>(row)), dst + seg * 1024);
        }
    };

    // this lane's key, and K/V as B operands (column = key, K-slots = dims)
    const int wk0 = k0 + 32 * w;
    const int key = wk0 + l32;
    const bool key_live = key < N;
    bf16x8 kf[D / 16], vf[D / 16];
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
        uint4 ku = make_uint4(0, 0, 0, 0), vu = ku;
        if (key_live) {
            ku = *reinterpret_cast<const uint4*>(Kh + (size_t)key * D + 16 * ks + 8 * g);
            vu = *reinterpret_cast<const uint4*>(Vh + (size_t)key * D + 16 * ks + 8 * g);
        }
        kf[ks] = as_bf16x8(ku);
        vf[ks] = as_bf16x8(vu);
    }

    // per-lane LDS offsets.  Row-major chunk reads: row 32*b + l32, chunk 2*ks + g.
    int rd_off[D / 16];
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) rd_off[ks] = l32 * ROWB + 16 * ((2 * ks + g) ^ bwd_swz<D>(l32));
    // Transposed reads: rows rt + 4*u (u selects the 4-row group), columns
    // 32*mb + ct .. +3.  The swizzle depends on (row % 16), i.e. on rt and on
    // the 4-row group index modulo 4.
    const int rt = (lane & 15) >> 2;
    const int ct = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    auto tr_off = [&](int row, int col) __attribute__((always_inline)) -> int {
        return row * ROWB + 16 * ((col >> 3) ^ bwd_swz<D>(row)) + 2 * (col & 7);
    };

    f32x16 dvt[D / 32], dkt[D / 32];
#pragma unroll
    for (int mb = 0; mb < D / 32; ++mb) {
        dvt[mb] = zero16();
        dkt[mb] = zero16();
    }

    const int nqt = (N + BR - 1) / BR;
    const int qt_begin = CAUSAL ? (k0 / BR) : 0;

    // LSE (wave 0) and D (wave 1) of the query tile starting at row r0, one
    // row per lane; rows past the end are clamped (and masked later)
    auto issue_stats = [&](int r0, float* ldst, float* ddst) __attribute__((always_inline)) {
        const int row = min(r0 + lane, N - 1);
        if (w == 0) g2lds4(LSEh + row, ldst);
        if (w == 1) g2lds4(Dh + row, ddst);
    };

    // buffer layout: Q tile | dO tile | LSE[BR] | D[BR]
    auto fill = [&](int r0, char* b) __attribute__((always_inline)) {
        issue(Qh, r0, b, w * QSPW, QSPW);
        issue(dOh, r0, b + QTB, w * QSPW, QSPW);
        issue_stats(r0, reinterpret_cast<float*>(b + 2 * QTB), reinterpret_cast<float*>(b + 2 * QTB + 4 * BR));
    };

    // prologue: K tile (once) and the first query tile
    issue(Kh, k0, kbuf, w * KSPW, KSPW);
    if (qt_begin < nqt) fill(qt_begin * BR, buf0);
    FA_WAIT_VMCNT(0);

    auto tile = [&](int qt, const char* cur, char* nxt) __attribute__((always_inline)) {
        const char* qs = cur;
        const char* os = cur + QTB;
        const float* ls = reinterpret_cast<const float*>(cur + 2 * QTB);
        const float* ds_ = reinterpret_cast<const float*>(cur + 2 * QTB + 4 * BR);
        const int q0 = qt * BR;
        // copies of this tile have landed (the atomics of the previous tile,
        // issued after them, may still be in flight); every wave is done with
        // the previous tile, so its buffers may be refilled
        FA_WAIT_VMCNT(ATOMICS);
        __builtin_amdgcn_s_barrier();
        if (qt + 1 < nqt) fill(q0 + BR, nxt);

        const bool wave_dead = (CAUSAL && wk0 > q0 + BR - 1) || wk0 >= N;
        if (wave_dead) {
            // this wave's keys see none of the tile's queries: dS = 0
#pragma unroll
            for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    dss[(32 * qb + 8 * (r >> 2) + 4 * g + (r & 3)) * DSS + 32 * w + l32] = (__bf16)0.f;
        } else {
            // LSE and D of this lane's 16 query rows per block (runs of 4)
            float4 lse4[NQB][4], dd4[NQB][4];
#pragma unroll
            for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
                for (int rb = 0; rb < 4; ++rb) {
                    lse4[qb][rb] = *reinterpret_cast<const float4*>(ls + 32 * qb + 8 * rb + 4 * g);
                    dd4[qb][rb] = *reinterpret_cast<const float4*>(ds_ + 32 * qb + 8 * rb + 4 * g);
                }

            f32x16 sP[NQB], dP[NQB];
#pragma unroll
            for (int qb = 0; qb < NQB; ++qb) {
                sP[qb] = zero16();
                dP[qb] = zero16();
            }
#pragma unroll
            for (int ks = 0; ks < D / 16; ++ks)
#pragma unroll
                for (int qb = 0; qb < NQB; ++qb) {
                    const bf16x8 aq = *reinterpret_cast<const bf16x8*>(qs + 32 * qb * ROWB + rd_off[ks]);
                    sP[qb] = mfma_bf16(aq, kf[ks], sP[qb]);
                    const bf16x8 ad = *reinterpret_cast<const bf16x8*>(os + 32 * qb * ROWB + rd_off[ks]);
                    dP[qb] = mfma_bf16(ad, vf[ks], dP[qb]);
                }
            // P = 2^(c S - LSE log2 e), masked; dS = P (dP - D)
            const bool need_mask = (k0 + BC > N) || (q0 + BR > N) || (CAUSAL && wk0 + 31 > q0);
#pragma unroll
            for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
                for (int rb = 0; rb < 4; ++rb) {
                    const float lv[4] = {lse4[qb][rb].x, lse4[qb][rb].y, lse4[qb][rb].z, lse4[qb][rb].w};
                    const float dv[4] = {dd4[qb][rb].x, dd4[qb][rb].y, dd4[qb][rb].z, dd4[qb][rb].w};
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        const int r = 4 * rb + t;
                        const int qrow = q0 + 32 * qb + 8 * rb + 4 * g + t;
                        float p = exp2_fast(fmaf(sP[qb][r], c, -lv[t] * kLog2e));
                        if (need_mask && (!key_live || qrow >= N || (CAUSAL && key > qrow))) p = 0.f;
                        sP[qb][r] = p;
                        dP[qb][r] = p * (dP[qb][r] - dv[t]);
                    }
                }
            // dV^T += dO^T P ; dK^T += Q^T dS  (K-slots = queries, permuted as
            // in the C layout; the transposed reads follow the same order)
#pragma unroll
            for (int ks = 0; ks < BR / 16; ++ks) {
                const int qb = ks >> 1, h = ks & 1;
                uint32_t pk[4], sk[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    pk[j] = pack_bf16x2(sP[qb][8 * h + 2 * j], sP[qb][8 * h + 2 * j + 1]);
                    sk[j] = pack_bf16x2(dP[qb][8 * h + 2 * j], dP[qb][8 * h + 2 * j + 1]);
                }
                const bf16x8 pb = as_bf16x8(make_uint4(pk[0], pk[1], pk[2], pk[3]));
                const bf16x8 sb = as_bf16x8(make_uint4(sk[0], sk[1], sk[2], sk[3]));
                const int row_lo = 16 * ks + 4 * g + rt;       // queries of K-slots j = 0..3
#pragma unroll
                for (int mb = 0; mb < D / 32; ++mb) {
                    const int col = 32 * mb + ct;
                    const uint2 dlo = lds_read_tr16x4(os + tr_off(row_lo, col));
                    const uint2 dhi = lds_read_tr16x4(os + tr_off(row_lo + 8, col));
                    dvt[mb] = mfma_bf16(as_bf16x8(make_uint4(dlo.x, dlo.y, dhi.x, dhi.y)), pb, dvt[mb]);
                    const uint2 qlo = lds_read_tr16x4(qs + tr_off(row_lo, col));
                    const uint2 qhi = lds_read_tr16x4(qs + tr_off(row_lo + 8, col));
                    dkt[mb] = mfma_bf16(as_bf16x8(make_uint4(qlo.x, qlo.y, qhi.x, qhi.y)), sb, dkt[mb]);
                }
            }
            // dS -> LDS as [query][key] bf16 for dQ
#pragma unroll
            for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    dss[(32 * qb + 8 * (r >> 2) + 4 * g + (r & 3)) * DSS + 32 * w + l32] = (__bf16)dP[qb][r];
        }
        FA_WAIT_LGKM0();
        __builtin_amdgcn_s_barrier();

        // dQ_tile += dS K : DQ_UNITS 32x32 output blocks shared by the waves.
        // K-slots are keys in natural order; the K^T operand is read
        // transposed from the row-major K tile.
#pragma unroll
        for (int u0 = 0; u0 < DQ_PER_WAVE; ++u0) {
            const int u = u0 * 4 + w;
            const int qb = u / (D / 32), nb = u % (D / 32);
            f32x16 acc = zero16();
#pragma unroll
            for (int ks = 0; ks < BC / 16; ++ks) {
                const bf16x8 a = *reinterpret_cast<const bf16x8*>(dss + (32 * qb + l32) * DSS + 16 * ks + 8 * g);
                const int row = 16 * ks + 8 * g + rt;
                const int col = 32 * nb + ct;
                const uint2 lo = lds_read_tr16x4(kbuf + tr_off(row, col));
                const uint2 hi = lds_read_tr16x4(kbuf + tr_off(row + 4, col));
                acc = mfma_bf16(a, as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y)), acc);
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = q0 + 32 * qb + 8 * (r >> 2) + 4 * g + (r & 3);
                if (row < N) unsafeAtomicAdd(dQh + (size_t)row * D + 32 * nb + l32, acc[r]);
            }
        }
    };

    for (int qt = qt_begin; qt < nqt; qt += 2) {
        tile(qt, buf0, buf1);
        if (qt + 1 < nqt) tile(qt + 1, buf1, buf0);
    }

    // dV = (dV^T)^T, dK = scale (dK^T)^T: lane holds key `key`, dims in runs of 4
    if (key_live) {
        __bf16* dvrow = dV + hoff + (size_t)key * D;
        __bf16* dkrow = dK + hoff + (size_t)key * D;
#pragma unroll
        for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
            for (int rb = 0; rb < 4; ++rb) {
                const int d0 = 32 * mb + 8 * rb + 4 * g;
                *reinterpret_cast<uint2*>(dvrow + d0) =
                    make_uint2(pack_bf16x2(dvt[mb][4 * rb], dvt[mb][4 * rb + 1]),
                               pack_bf16x2(dvt[mb][4 * rb + 2], dvt[mb][4 * rb + 3]));
                *reinterpret_cast<uint2*>(dkrow + d0) =
                    make_uint2(pack_bf16x2(scale * dkt[mb][4 * rb], scale * dkt[mb][4 * rb + 1]),
                               pack_bf16x2(scale * dkt[mb][4 * rb + 2], scale * dkt[mb][4 * rb + 3]));
            }
    }
}

// ---------------------------------------------------------------------------
// 3. dQ = scale * accumulator -> bf16 (8 elements per thread)
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256)
bwd_dq_kernel(const float* __restrict__ acc, __bf16* __restrict__ dq, long long n8, float scale) {
    const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
    if (i >= n8) return;
    const float4 a = *reinterpret_cast<const float4*>(acc + 8 * i);
    const float4 b = *reinterpret_cast<const float4*>(acc + 8 * i + 4);
    *reinterpret_cast<uint4*>(dq + 8 * i) =
        make_uint4(pack_bf16x2(scale * a.x, scale * a.y), pack_bf16x2(scale * a.z, scale * a.w),
                   pack_bf16x2(scale * b.x, scale * b.y), pack_bf16x2(scale * b.z, scale * b.w));
}

template <int D, bool CAUSAL>
hipError_t launch_main(const BwdArgs& a) {
    const int BH = a.B * a.H;
    const int nkt = (a.N + BWD_BC - 1) / BWD_BC;
    hipLaunchKernelGGL((bwd_main_kernel<D, CAUSAL>), dim3((unsigned)(nkt * BH)), dim3(BWD_THREADS), 0,
                       (hipStream_t)a.stream, (const __bf16*)a.q, (const __bf16*)a.k, (const __bf16*)a.v,
                       (const __bf16*)a.dout, a.lse, a.delta, a.dq_acc, (__bf16*)a.dk, (__bf16*)a.dv, BH, a.N,
                       a.scale * kLog2e, a.scale);
    return hipGetLastError();
}

template <int D>
hipError_t launch_d(const BwdArgs& a) {
    hipStream_t st = (hipStream_t)a.stream;
    const long long rows = (long long)a.B * a.H * a.N;
    const long long prep_threads = rows * (D / 8);
    const unsigned prep_blocks = (unsigned)((prep_threads + 255) / 256);
    if (a.o_bf16)
        hipLaunchKernelGGL((bwd_prep_kernel<D, true>), dim3(prep_blocks), dim3(256), 0, st, a.o,
                           (const __bf16*)a.dout, a.delta, a.dq_acc, rows);
    else
        hipLaunchKernelGGL((bwd_prep_kernel<D, false>), dim3(prep_blocks), dim3(256), 0, st, a.o,
                           (const __bf16*)a.dout, a.delta, a.dq_acc, rows);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    e = a.causal ? launch_main<D, true>(a) : launch_main<D, false>(a);
    if (e != hipSuccess) return e;
    const long long n8 = rows * D / 8;
    hipLaunchKernelGGL(bwd_dq_kernel, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, st, a.dq_acc,
                       (__bf16*)a.dq, n8, a.scale);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd(const BwdArgs& a) {
    const long long rows = (long long)a.B * a.H * a.N;
    if (rows * (a.d / 8) / 256 + 1 > 0x7fffffffLL) return hipErrorInvalidValue;
    return a.d == 64 ? launch_d<64>(a) : launch_d<128>(a);
}

}  // namespace fa
