// fa_fwd.hip -- fused exact-attention forward for gfx950.
//
// One workgroup owns one tile of BR query rows of one (batch, head) and
// streams that head's K/V tiles through LDS, keeping the running row maximum,
// the running sum of exponentials and the unnormalised output in registers
// (online softmax: "FlashAttention (EL)", sections on tiling and on online
// softmax; "Flash Attention: Ako transformery ...", section 2).  QK^T,
// masking, softmax and PV are fused; only O and the per-row LSE are written
// (same Greek page, section on fusing all operations into one kernel).  Work
// is split over query tiles as well as heads so that small-batch long
// sequences fill the chip ("Flash Attention uitgelegd", FA2 section on
// parallelism over the sequence length).
//
// bf16 path (d = 64 or 128): four waves, 32 query rows each.  Per key tile
// of BC = 64 keys a wave computes S^T = K Q^T (keys x queries) with
// v_mfma_f32_32x32x16_bf16: K comes from LDS, Q^T stays in registers for the
// whole kernel.  In the C layout each lane then holds one query row and 16 of
// the tile's keys, so row max and row sum are in-lane work plus one exchange
// with lane ^ 32.  The probabilities, rounded to bf16, are already a valid B
// operand of O^T += V^T P^T, given V^T staged in LDS with the matching key
// permutation; O^T again gives each lane one query row.  The scale is folded
// into the exp2 argument and O is normalised once at the end (the FA2 point
// about minimising non-matmul work).
//
// fp32 path: same structure on v_mfma_f32_32x32x2_f32 with BC = 32; V needs no
// transpose because each fp32 K-slot holds a single key.
#include "fa_common.hpp"
#include "fa_internal.hpp"

namespace fa {

namespace {

constexpr int FWD_BR = 128;     // query rows per workgroup (4 waves x 32)
constexpr int FWD_BC = 64;      // keys per K/V tile, bf16 path
constexpr int FWD_BC32 = 32;    // keys per K/V tile, fp32 path
constexpr int FWD_THREADS = 256;

// Map the flat block id to (head, query tile).  Consecutive ids are
// consecutive heads, so every head's tiles land on the same XCD when the head
// count is a multiple of 8 (the hardware deals blocks round-robin to the 8
// XCDs), and with a causal mask the most expensive (last) query tiles of all
// heads are issued first.
__device__ __forceinline__ void fwd_tile_of(int bid, int BH, int nqt, bool causal,
                                            int& bh, int& qt) {
    bh = bid % BH;
    const int t = bid / BH;
    qt = causal ? (nqt - 1 - t) : t;
}

template <int D, bool CAUSAL, bool OUT_BF16>
__global__ void __launch_bounds__(FWD_THREADS)
fwd_bf16_kernel(const __bf16* __restrict__ Q, const __bf16* __restrict__ K,
                const __bf16* __restrict__ V, void* __restrict__ O, float* __restrict__ LSE,
                int BH, int N, int nqt, float c /* scale * log2(e) */) {
    constexpr int BR = FWD_BR, BC = FWD_BC;
    constexpr int KS = D + 8;      // LDS row stride (bf16) of the K tile
    constexpr int VS = BC + 8;     // LDS row stride (bf16) of the V^T tile
    constexpr int KCH = BC * D / 8;                // 16-byte chunks in a K tile
    constexpr int KPT = KCH / FWD_THREADS;         // chunks per thread
    constexpr int VBLK = (BC / 4) * (D / 8);       // 4-key x 8-dim blocks in a V tile
    constexpr int VPT = (VBLK + FWD_THREADS - 1) / FWD_THREADS;
    static_assert(KCH % FWD_THREADS == 0, "K tile must split evenly");

    __shared__ __attribute__((aligned(16))) __bf16 Ks[BC * KS];
    __shared__ __attribute__((aligned(16))) __bf16 Vt[D * VS];

    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const int l32 = lane & 31, g = lane >> 5;

    int bh, qt;
    fwd_tile_of(blockIdx.x, BH, nqt, CAUSAL, bh, qt);
    const int q0 = qt * BR;
    const size_t hoff = (size_t)bh * (size_t)N * D;
    const __bf16* Qh = Q + hoff;
    const __bf16* Kh = K + hoff;
    const __bf16* Vh = V + hoff;

    // Q^T fragment: B operand of S^T = K Q^T, column = query row of this lane.
    const int qrow = q0 + 32 * w + l32;
    bf16x8 qf[D / 16];
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
        uint4 u = make_uint4(0, 0, 0, 0);
        if (qrow < N) u = *reinterpret_cast<const uint4*>(Qh + (size_t)qrow * D + 16 * ks + 8 * g);
        qf[ks] = as_bf16x8(u);
    }

    f32x16 oacc[D / 32];
#pragma unroll
    for (int mb = 0; mb < D / 32; ++mb) oacc[mb] = zero16();
    float m_run = -INFINITY;   // running max of scale*log2(e)*s over the row
    float l_run = 0.f;         // this lane's share of the running sum

    const int kv_end = CAUSAL ? min(N, q0 + BR) : N;
    const int nkt = (kv_end + BC - 1) / BC;

    uint4 kreg[KPT];
    uint4 vreg[VPT][4];

    auto load_tile = [&](int kt) {
        const int kv0 = kt * BC;
#pragma unroll
        for (int i = 0; i < KPT; ++i) {
            const int ch = tid + FWD_THREADS * i;
            const int row = ch / (D / 8), c8 = ch % (D / 8);
            uint4 u = make_uint4(0, 0, 0, 0);
            if (kv0 + row < N) u = *reinterpret_cast<const uint4*>(Kh + (size_t)(kv0 + row) * D + 8 * c8);
            kreg[i] = u;
        }
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            const int blk = tid + FWD_THREADS * i;
            const int kq = blk % (BC / 4), dc = blk / (BC / 4);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int key = kv0 + 4 * kq + r;
                uint4 u = make_uint4(0, 0, 0, 0);
                if (blk < VBLK && key < N) u = *reinterpret_cast<const uint4*>(Vh + (size_t)key * D + 8 * dc);
                vreg[i][r] = u;
            }
        }
    };
    auto store_tile = [&]() {
#pragma unroll
        for (int i = 0; i < KPT; ++i) {
            const int ch = tid + FWD_THREADS * i;
            const int row = ch / (D / 8), c8 = ch % (D / 8);
            *reinterpret_cast<uint4*>(Ks + row * KS + 8 * c8) = kreg[i];
        }
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            const int blk = tid + FWD_THREADS * i;
            if (blk < VBLK) {
                const int kq = blk % (BC / 4), dc = blk / (BC / 4);
                const int pos = perm16(4 * kq);
#pragma unroll
                for (int cc = 0; cc < 8; ++cc)
                    *reinterpret_cast<uint2*>(Vt + (8 * dc + cc) * VS + pos) =
                        column4(vreg[i][0], vreg[i][1], vreg[i][2], vreg[i][3], cc);
            }
        }
    };

    if (nkt > 0) load_tile(0);
    const int wrow0 = q0 + 32 * w;
    for (int kt = 0; kt < nkt; ++kt) {
        __syncthreads();
        store_tile();
        __syncthreads();
        if (kt + 1 < nkt) load_tile(kt + 1);

        const int kv0 = kt * BC;
        if (wrow0 >= N) continue;                       // padding wave
        if (CAUSAL && kv0 > wrow0 + 31) continue;       // tile entirely above the diagonal

        // S^T = K Q^T : two 32-key blocks
        f32x16 s[BC / 32];
#pragma unroll
        for (int kb = 0; kb < BC / 32; ++kb) {
            s[kb] = zero16();
#pragma unroll
            for (int ks = 0; ks < D / 16; ++ks) {
                const bf16x8 a = *reinterpret_cast<const bf16x8*>(Ks + (32 * kb + l32) * KS + 16 * ks + 8 * g);
                s[kb] = mfma_bf16(a, qf[ks], s[kb]);
            }
        }

        const bool need_mask = (kv0 + BC > N) || (CAUSAL && kv0 + BC - 1 > wrow0);
        if (need_mask) {
#pragma unroll
            for (int kb = 0; kb < BC / 32; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = kv0 + 32 * kb + 8 * (r >> 2) + 4 * g + (r & 3);
                    if (key >= N || (CAUSAL && key > qrow)) s[kb][r] = -INFINITY;
                }
        }

        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < BC / 32; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
        mx = xor32_max(mx);
        const float m_new = fmaxf(m_run, mx * c);
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
        const float alpha = exp2_fast(m_run - m_use);
        m_run = m_new;

        // P (bf16) laid out as the B operand of O^T += V^T P^T
        bf16x8 pb[BC / 16];
        float psum = 0.f;
#pragma unroll
        for (int kb = 0; kb < BC / 32; ++kb)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                uint32_t pk[4];
#pragma unroll
                for (int j = 0; j < 8; j += 2) {
                    const float p0 = exp2_fast(fmaf(s[kb][8 * h + j], c, -m_use));
                    const float p1 = exp2_fast(fmaf(s[kb][8 * h + j + 1], c, -m_use));
                    psum += p0 + p1;
                    pk[j / 2] = pack_bf16x2(p0, p1);
                }
                pb[2 * kb + h] = as_bf16x8(make_uint4(pk[0], pk[1], pk[2], pk[3]));
            }
        l_run = l_run * alpha + psum;
#pragma unroll
        for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[mb][r] *= alpha;

        // O^T += V^T P^T
#pragma unroll
        for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
            for (int ks = 0; ks < BC / 16; ++ks) {
                const bf16x8 a = *reinterpret_cast<const bf16x8*>(Vt + (32 * mb + l32) * VS + 16 * ks + 8 * g);
                oacc[mb] = mfma_bf16(a, pb[ks], oacc[mb]);
            }
    }

    const float l_tot = xor32_sum(l_run);
    if (qrow < N) {
        const float inv = (l_tot > 0.f) ? 1.f / l_tot : 0.f;
        const size_t orow = (size_t)bh * N * D + (size_t)qrow * D;
#pragma unroll
        for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
            for (int rb = 0; rb < 4; ++rb) {
                const int d0 = 32 * mb + 8 * rb + 4 * g;
                const float o0 = oacc[mb][4 * rb + 0] * inv, o1 = oacc[mb][4 * rb + 1] * inv;
                const float o2 = oacc[mb][4 * rb + 2] * inv, o3 = oacc[mb][4 * rb + 3] * inv;
                if (OUT_BF16) {
                    *reinterpret_cast<uint2*>(static_cast<__bf16*>(O) + orow + d0) =
                        make_uint2(pack_bf16x2(o0, o1), pack_bf16x2(o2, o3));
                } else {
                    *reinterpret_cast<float4*>(static_cast<float*>(O) + orow + d0) = make_float4(o0, o1, o2, o3);
                }
            }
        if (g == 0)
            LSE[(size_t)bh * N + qrow] = (l_tot > 0.f) ? m_run * kLn2 + __logf(l_tot) : -INFINITY;
    }
}

template <int D, bool CAUSAL>
__global__ void __launch_bounds__(FWD_THREADS)
fwd_f32_kernel(const float* __restrict__ Q, const float* __restrict__ K,
               const float* __restrict__ V, float* __restrict__ O, float* __restrict__ LSE,
               int BH, int N, int nqt, float c) {
    constexpr int BR = FWD_BR, BC = FWD_BC32;
    constexpr int KS = D + 1;      // odd stride: column reads hit distinct banks
    constexpr int VS = D;
    constexpr int CH = BC * D / 4;                 // 16-byte chunks per tile
    constexpr int CPT = CH / FWD_THREADS;
    static_assert(CH % FWD_THREADS == 0, "tile must split evenly");

    __shared__ __attribute__((aligned(16))) float Ks[BC * KS];
    __shared__ __attribute__((aligned(16))) float Vs[BC * VS];

    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const int l32 = lane & 31, g = lane >> 5;

    int bh, qt;
    fwd_tile_of(blockIdx.x, BH, nqt, CAUSAL, bh, qt);
    const int q0 = qt * BR;
    const size_t hoff = (size_t)bh * (size_t)N * D;
    const float* Qh = Q + hoff;
    const float* Kh = K + hoff;
    const float* Vh = V + hoff;

    const int qrow = q0 + 32 * w + l32;
    float qf[D / 2];
#pragma unroll
    for (int ks = 0; ks < D / 2; ++ks) qf[ks] = (qrow < N) ? Qh[(size_t)qrow * D + 2 * ks + g] : 0.f;

    f32x16 oacc[D / 32];
#pragma unroll
    for (int mb = 0; mb < D / 32; ++mb) oacc[mb] = zero16();
    float m_run = -INFINITY, l_run = 0.f;

    const int kv_end = CAUSAL ? min(N, q0 + BR) : N;
    const int nkt = (kv_end + BC - 1) / BC;
    const int wrow0 = q0 + 32 * w;

    for (int kt = 0; kt < nkt; ++kt) {
        const int kv0 = kt * BC;
        __syncthreads();
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const int ch = tid + FWD_THREADS * i;
            const int row = ch / (D / 4), c4 = ch % (D / 4);
            float4 kk = make_float4(0.f, 0.f, 0.f, 0.f), vv = kk;
            if (kv0 + row < N) {
                kk = *reinterpret_cast<const float4*>(Kh + (size_t)(kv0 + row) * D + 4 * c4);
                vv = *reinterpret_cast<const float4*>(Vh + (size_t)(kv0 + row) * D + 4 * c4);
            }
            float* kd = Ks + row * KS + 4 * c4;
            kd[0] = kk.x; kd[1] = kk.y; kd[2] = kk.z; kd[3] = kk.w;
            *reinterpret_cast<float4*>(Vs + row * VS + 4 * c4) = vv;
        }
        __syncthreads();
        if (wrow0 >= N) continue;
        if (CAUSAL && kv0 > wrow0 + 31) continue;

        f32x16 s = zero16();
#pragma unroll
        for (int ks = 0; ks < D / 2; ++ks) s = mfma_f32(Ks[l32 * KS + 2 * ks + g], qf[ks], s);

        if ((kv0 + BC > N) || (CAUSAL && kv0 + BC - 1 > wrow0)) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = kv0 + 8 * (r >> 2) + 4 * g + (r & 3);
                if (key >= N || (CAUSAL && key > qrow)) s[r] = -INFINITY;
            }
        }
        float mx = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[r]);
        mx = xor32_max(mx);
        const float m_new = fmaxf(m_run, mx * c);
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
        const float alpha = exp2_fast(m_run - m_use);
        m_run = m_new;
        float psum = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            s[r] = exp2_fast(fmaf(s[r], c, -m_use));
            psum += s[r];
        }
        l_run = l_run * alpha + psum;
#pragma unroll
        for (int mb = 0; mb < D / 32; ++mb) {
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[mb][r] *= alpha;
            // K-slot r of this lane = key 8*(r/4) + 4*g + r%4, matching C register r of S^T
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = 8 * (r >> 2) + 4 * g + (r & 3);
                oacc[mb] = mfma_f32(Vs[key * VS + 32 * mb + l32], s[r], oacc[mb]);
            }
        }
    }

    const float l_tot = xor32_sum(l_run);
    if (qrow < N) {
        const float inv = (l_tot > 0.f) ? 1.f / l_tot : 0.f;
        float* orow = O + (size_t)bh * N * D + (size_t)qrow * D;
#pragma unroll
        for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
            for (int rb = 0; rb < 4; ++rb) {
                const int d0 = 32 * mb + 8 * rb + 4 * g;
                *reinterpret_cast<float4*>(orow + d0) =
                    make_float4(oacc[mb][4 * rb] * inv, oacc[mb][4 * rb + 1] * inv,
                                oacc[mb][4 * rb + 2] * inv, oacc[mb][4 * rb + 3] * inv);
            }
        if (g == 0)
            LSE[(size_t)bh * N + qrow] = (l_tot > 0.f) ? m_run * kLn2 + __logf(l_tot) : -INFINITY;
    }
}

template <int D, bool CAUSAL, bool OUT_BF16>
hipError_t launch_bf16(const FwdArgs& a) {
    const int BH = a.B * a.H;
    const int nqt = (a.N + FWD_BR - 1) / FWD_BR;
    const dim3 grid((unsigned)(nqt * BH)), block(FWD_THREADS);
    hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL, OUT_BF16>), grid, block, 0, (hipStream_t)a.stream,
                       (const __bf16*)a.q, (const __bf16*)a.k, (const __bf16*)a.v, a.o, a.lse, BH, a.N, nqt,
                       a.scale * kLog2e);
    return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t launch_f32(const FwdArgs& a) {
    const int BH = a.B * a.H;
    const int nqt = (a.N + FWD_BR - 1) / FWD_BR;
    const dim3 grid((unsigned)(nqt * BH)), block(FWD_THREADS);
    hipLaunchKernelGGL((fwd_f32_kernel<D, CAUSAL>), grid, block, 0, (hipStream_t)a.stream,
                       (const float*)a.q, (const float*)a.k, (const float*)a.v, (float*)a.o, a.lse, BH, a.N,
                       nqt, a.scale * kLog2e);
    return hipGetLastError();
}

template <int D>
hipError_t dispatch_d(const FwdArgs& a) {
    if (!a.in_bf16) return a.causal ? launch_f32<D, true>(a) : launch_f32<D, false>(a);
    if (a.out_bf16) return a.causal ? launch_bf16<D, true, true>(a) : launch_bf16<D, false, true>(a);
    return a.causal ? launch_bf16<D, true, false>(a) : launch_bf16<D, false, false>(a);
}

}  // namespace

hipError_t launch_fwd(const FwdArgs& a) {
    if ((long long)((a.N + FWD_BR - 1) / FWD_BR) * a.B * a.H > 0x7fffffffLL) return hipErrorInvalidValue;
    return a.d == 64 ? dispatch_d<64>(a) : dispatch_d<128>(a);
}

}  // namespace fa
