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
//                 32 keys each).  K and V of the tile stay in registers; the
//                 workgroup walks the query tiles (BR = 64 rows) that can see
//                 its keys, staging Q and dO in LDS both row-major and
//                 transposed.  dK^T and dV^T accumulate in registers; dS goes
//                 through LDS so that all four waves contribute to
//                 dQ_i += dS K_j, which is added into the fp32 accumulator with
//                 global atomics.
//   3. bwd_dq:    dQ = scale * accumulator, rounded to bf16.
//
// Layout trick (as in the forward): S is computed with queries as MFMA rows
// and keys as columns, so each lane holds one key and 16 queries; those
// registers are directly the K-slot-ordered B operands of dV^T = dO^T P and
// dK^T = Q^T dS when Q^T and dO^T are staged with the matching query
// permutation.
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
template <int D>
struct BwdSmem {
    static constexpr int RS = D + 8;          // row-major [BR][D] stride
    static constexpr int TS = BWD_BR + 8;     // transposed [D][BR] stride
    static constexpr int KTS = BWD_BC + 8;    // K^T [D][BC] stride
    static constexpr int DSS = BWD_BC + 8;    // dS [BR][BC] stride
    __bf16 q[BWD_BR * RS];
    __bf16 qt[D * TS];
    __bf16 dO[BWD_BR * RS];
    __bf16 dOt[D * TS];
    __bf16 kt[D * KTS];
    __bf16 ds[BWD_BR * DSS];
    float lse[BWD_BR];
    float dd[BWD_BR];
};

template <int D, bool CAUSAL>
__global__ void __launch_bounds__(BWD_THREADS)
bwd_main_kernel(const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
                const __bf16* __restrict__ dO, const float* __restrict__ LSE,
                const float* __restrict__ delta, float* __restrict__ dq_acc, __bf16* __restrict__ dK,
                __bf16* __restrict__ dV, int BH, int N, float c /* scale*log2e */, float scale) {
    using SM = BwdSmem<D>;
    constexpr int BR = BWD_BR, BC = BWD_BC;
    constexpr int RS = SM::RS, TS = SM::TS, KTS = SM::KTS, DSS = SM::DSS;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
    SM& sm = *reinterpret_cast<SM*>(smem_raw);

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

    // K^T of the whole tile in LDS (natural key order), B operand of dQ = dS K
    {
        constexpr int NBLK = (BC / 4) * (D / 8);
#pragma unroll
        for (int i = 0; i < (NBLK + BWD_THREADS - 1) / BWD_THREADS; ++i) {
            const int blk = tid + BWD_THREADS * i;
            if (blk < NBLK) {
                const int kq = blk % (BC / 4), dc = blk / (BC / 4);
                uint4 r[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int kk = k0 + 4 * kq + j;
                    r[j] = make_uint4(0, 0, 0, 0);
                    if (kk < N) r[j] = *reinterpret_cast<const uint4*>(Kh + (size_t)kk * D + 8 * dc);
                }
#pragma unroll
                for (int cc = 0; cc < 8; ++cc)
                    *reinterpret_cast<uint2*>(sm.kt + (8 * dc + cc) * KTS + 4 * kq) = column4(r[0], r[1], r[2], r[3], cc);
            }
        }
    }

    f32x16 dvt[D / 32], dkt[D / 32];
#pragma unroll
    for (int mb = 0; mb < D / 32; ++mb) {
        dvt[mb] = zero16();
        dkt[mb] = zero16();
    }

    const int nqt = (N + BR - 1) / BR;
    const int qt_begin = CAUSAL ? (k0 / BR) : 0;
    for (int qt = qt_begin; qt < nqt; ++qt) {
        const int q0 = qt * BR;
        __syncthreads();
        // stage Q and dO: 4-row x 8-dim blocks, row-major and transposed (query-permuted)
        {
            constexpr int NBLK = (BR / 4) * (D / 8);
#pragma unroll
            for (int i = 0; i < (NBLK + BWD_THREADS - 1) / BWD_THREADS; ++i) {
                const int blk = tid + BWD_THREADS * i;
                if (blk < NBLK) {
                    const int rq = blk % (BR / 4), dc = blk / (BR / 4);
                    uint4 qr[4], dr[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int row = q0 + 4 * rq + j;
                        qr[j] = make_uint4(0, 0, 0, 0);
                        dr[j] = qr[j];
                        if (row < N) {
                            qr[j] = *reinterpret_cast<const uint4*>(Qh + (size_t)row * D + 8 * dc);
                            dr[j] = *reinterpret_cast<const uint4*>(dOh + (size_t)row * D + 8 * dc);
                        }
                        *reinterpret_cast<uint4*>(sm.q + (4 * rq + j) * RS + 8 * dc) = qr[j];
                        *reinterpret_cast<uint4*>(sm.dO + (4 * rq + j) * RS + 8 * dc) = dr[j];
                    }
                    const int pos = perm16(4 * rq);
#pragma unroll
                    for (int cc = 0; cc < 8; ++cc) {
                        *reinterpret_cast<uint2*>(sm.qt + (8 * dc + cc) * TS + pos) = column4(qr[0], qr[1], qr[2], qr[3], cc);
                        *reinterpret_cast<uint2*>(sm.dOt + (8 * dc + cc) * TS + pos) = column4(dr[0], dr[1], dr[2], dr[3], cc);
                    }
                }
            }
            if (tid < BR) {
                const int row = q0 + tid;
                // rows past the end get LSE = +inf, so their P is exactly 0
                sm.lse[tid] = (row < N) ? LSEh[row] * kLog2e : INFINITY;
                sm.dd[tid] = (row < N) ? Dh[row] : 0.f;
            }
        }
        __syncthreads();

        const bool wave_dead = (!CAUSAL ? false : (wk0 > q0 + BR - 1)) || wk0 >= N;
        if (wave_dead) {
            // this wave's keys see none of the tile's queries: dS = 0
#pragma unroll
            for (int qb = 0; qb < BR / 32; ++qb)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    sm.ds[(32 * qb + 8 * (r >> 2) + 4 * g + (r & 3)) * DSS + 32 * w + l32] = (__bf16)0.f;
        } else {
            f32x16 sP[BR / 32], dP[BR / 32];
#pragma unroll
            for (int qb = 0; qb < BR / 32; ++qb) {
                sP[qb] = zero16();
                dP[qb] = zero16();
#pragma unroll
                for (int ks = 0; ks < D / 16; ++ks) {
                    const bf16x8 aq = *reinterpret_cast<const bf16x8*>(sm.q + (32 * qb + l32) * RS + 16 * ks + 8 * g);
                    sP[qb] = mfma_bf16(aq, kf[ks], sP[qb]);
                    const bf16x8 ad = *reinterpret_cast<const bf16x8*>(sm.dO + (32 * qb + l32) * RS + 16 * ks + 8 * g);
                    dP[qb] = mfma_bf16(ad, vf[ks], dP[qb]);
                }
            }
            // P = 2^(c S - LSE*log2e), masked; dS = P (dP - D)
            const bool need_mask = (k0 + BC > N) || (CAUSAL && wk0 + 31 > q0);
#pragma unroll
            for (int qb = 0; qb < BR / 32; ++qb)
#pragma unroll
                for (int rb = 0; rb < 4; ++rb) {
                    const int qi = 32 * qb + 8 * rb + 4 * g;
                    const float4 lse4 = *reinterpret_cast<const float4*>(sm.lse + qi);
                    const float4 dd4 = *reinterpret_cast<const float4*>(sm.dd + qi);
                    const float lv[4] = {lse4.x, lse4.y, lse4.z, lse4.w};
                    const float dv[4] = {dd4.x, dd4.y, dd4.z, dd4.w};
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        const int r = 4 * rb + t;
                        float p = exp2_fast(fmaf(sP[qb][r], c, -lv[t]));
                        if (need_mask && (!key_live || (CAUSAL && key > q0 + qi + t))) p = 0.f;
                        sP[qb][r] = p;
                        dP[qb][r] = p * (dP[qb][r] - dv[t]);
                    }
                }
            // dV^T += dO^T P ; dK^T += Q^T dS  (K-slots = queries, permuted)
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
#pragma unroll
                for (int mb = 0; mb < D / 32; ++mb) {
                    const bf16x8 ad = *reinterpret_cast<const bf16x8*>(sm.dOt + (32 * mb + l32) * TS + 16 * ks + 8 * g);
                    dvt[mb] = mfma_bf16(ad, pb, dvt[mb]);
                    const bf16x8 aq = *reinterpret_cast<const bf16x8*>(sm.qt + (32 * mb + l32) * TS + 16 * ks + 8 * g);
                    dkt[mb] = mfma_bf16(aq, sb, dkt[mb]);
                }
            }
            // dS -> LDS as [query][key] bf16 for dQ
#pragma unroll
            for (int qb = 0; qb < BR / 32; ++qb)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    sm.ds[(32 * qb + 8 * (r >> 2) + 4 * g + (r & 3)) * DSS + 32 * w + l32] = (__bf16)dP[qb][r];
        }
        __syncthreads();

        // dQ_tile += dS K : (BR/32) x (D/32) output blocks shared by the waves
        constexpr int UNITS = (BR / 32) * (D / 32);
#pragma unroll
        for (int u0 = 0; u0 < UNITS; u0 += BWD_THREADS / 64) {
            const int u = u0 + w;
            if (u < UNITS) {
                const int qb = u / (D / 32), nb = u % (D / 32);
                f32x16 acc = zero16();
#pragma unroll
                for (int ks = 0; ks < BC / 16; ++ks) {
                    const bf16x8 a = *reinterpret_cast<const bf16x8*>(sm.ds + (32 * qb + l32) * DSS + 16 * ks + 8 * g);
                    const bf16x8 b = *reinterpret_cast<const bf16x8*>(sm.kt + (32 * nb + l32) * KTS + 16 * ks + 8 * g);
                    acc = mfma_bf16(a, b, acc);
                }
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = q0 + 32 * qb + 8 * (r >> 2) + 4 * g + (r & 3);
                    if (row < N) unsafeAtomicAdd(dQh + (size_t)row * D + 32 * nb + l32, acc[r]);
                }
            }
        }
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
    const size_t smem = sizeof(BwdSmem<D>);
    auto kern = bwd_main_kernel<D, CAUSAL>;
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3((unsigned)(nkt * BH)), dim3(BWD_THREADS), smem, (hipStream_t)a.stream,
                       (const __bf16*)a.q, (const __bf16*)a.k, (const __bf16*)a.v, (const __bf16*)a.dout, a.lse,
                       a.delta, a.dq_acc, (__bf16*)a.dk, (__bf16*)a.dv, BH, a.N, a.scale * kLog2e, a.scale);
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
