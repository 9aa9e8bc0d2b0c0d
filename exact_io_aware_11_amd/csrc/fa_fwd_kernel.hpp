// fa_fwd_kernel.hpp -- the bf16 forward kernel template of fa_fwd.hip.
//
// Kept in a header so that the measurement probe library can instantiate the
// same kernel with its clock record switched on (CLOCK = true): wave 0 of each
// workgroup then writes the shader-clock cycles (s_memtime) and the constant
// 100 MHz reference (s_memrealtime) its workgroup took.  The library itself
// only instantiates CLOCK = false, whose code has no clock reads.
#pragma once

#include "fa_common.hpp"

namespace fa {

// Internal linkage on purpose: the library and the probe library each
// compile their own instantiations, and neither exports them.
namespace {

constexpr int FWD_BR = 128;     // query rows per workgroup (4 waves x 32)
// Keys per K/V tile of the bf16 path.  d = 64 takes 64-key tiles (four waves
// per SIMD either way).  d = 128 takes 32-key tiles: the smaller S and P bring
// the kernel to 166 registers and 32 KB of LDS, so three workgroups -- three
// waves per SIMD -- are resident per CU instead of two, which overlaps one
// wave's softmax with the others' products better than the larger tile's
// fewer barriers do.  d = 256 also takes 32-key tiles, so that S, P and the
// 256-column O accumulator fit the registers of two waves per SIMD.
template <int D>
constexpr int fwd_bc() { return D == 64 ? 64 : 32; }
// waves per SIMD the register budget is sized for
template <int D>
constexpr int fwd_waves() { return D == 64 ? 4 : D == 128 ? 3 : 2; }
constexpr int FWD_BC32 = 32;    // keys per K/V tile, fp32 path
// instruction schedule of the bf16 tile loop (measured best on MI355X)
constexpr int QK_AHEAD = 6;        // K-operand LDS reads kept ahead of the S MFMAs
constexpr int PV_AHEAD = 4;        // V^T operands read ahead of the O MFMAs
constexpr int FWD_THREADS = 256;

// K and V tiles live in LDS row-major without padding (2*D bytes per row) and
// are filled by direct global->LDS copies; bank conflicts are avoided by
// permuting the 16-byte chunks of each row with an XOR of the row index
// (k_swz for K, read one chunk per lane by 32 consecutive rows; v_swz for V,
// read with the transposing 8-byte read).
template <int D, bool CAUSAL, bool OUT_BF16, bool CLOCK = false>
__global__ void __launch_bounds__(FWD_THREADS) __attribute__((amdgpu_waves_per_eu(fwd_waves<D>())))
fwd_bf16_kernel(const __bf16* __restrict__ Q, const __bf16* __restrict__ K,
                const __bf16* __restrict__ V, void* __restrict__ O, float* __restrict__ LSE,
                int BH, int G, int N, int nqt, float c /* scale * log2(e) */,
                unsigned long long* __restrict__ clk /* CLOCK: 2 per workgroup */) {
    constexpr int BR = FWD_BR, BC = fwd_bc<D>();
    constexpr int ROWB = 2 * D;              // bytes per K/V row in LDS
    constexpr int CPR = D / 8;               // 16-byte chunks per row
    constexpr int TILEB = BC * ROWB;         // bytes per K (or V) tile
    constexpr int RPS = 1024 / ROWB;         // rows per 1 KiB copy segment
    constexpr int SPW = TILEB / 1024 / 4;    // copy segments per wave per tile
    constexpr int NKB = BC / 32;             // 32-key blocks per tile
    constexpr float P_MAX = 256.f;           // largest tile row sum kept without rescaling
    static_assert(SPW >= 1, "tile too small for four waves");

    // Two buffer pairs (K tile, V tile): the copies of tile kt+1 run while
    // tile kt is computed.  Four separate LDS objects let the compiler see
    // that the copies into one pair never alias the reads of the other, so it
    // does not wait for them before reading.
    __shared__ __attribute__((aligned(1024))) char kb0[TILEB];
    __shared__ __attribute__((aligned(1024))) char kb1[TILEB];
    __shared__ __attribute__((aligned(1024))) char vb0[TILEB];
    __shared__ __attribute__((aligned(1024))) char vb1[TILEB];

    unsigned long long clk_t0 = 0, clk_r0 = 0;
    if constexpr (CLOCK) {
        clk_t0 = __builtin_amdgcn_s_memtime();
        clk_r0 = __builtin_amdgcn_s_memrealtime();
    }
    const int tid = threadIdx.x;
    // wave index made wave-uniform, so per-wave bounds and branches stay scalar
    const int lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, g = lane >> 5;

    int bh, qt;
    fwd_tile_of(blockIdx.x, BH, G, nqt, CAUSAL, bh, qt);
    const int q0 = qt * BR;
    const size_t hoff = (size_t)bh * (size_t)N * D;
    const size_t kvoff = (size_t)(bh / G) * (size_t)N * D;   // this head's K/V head
    const __bf16* Qh = Q + hoff;
    const __bf16* Kh = K + kvoff;
    const __bf16* Vh = V + kvoff;

    // Q^T fragment: B operand of S^T = K Q^T, column = query row of this lane.
    const int qrow = q0 + 32 * w + l32;
    bf16x8 qf[D / 16];
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
        uint4 u = make_uint4(0, 0, 0, 0);
        if (qrow < N) u = *reinterpret_cast<const uint4*>(Qh + (size_t)qrow * D + 16 * ks + 8 * g);
        qf[ks] = as_bf16x8(u);
    }

    const int kv_end = CAUSAL ? min(N, q0 + BR) : N;
    const int nkt = (kv_end + BC - 1) / BC;                 // tiles the workgroup streams
    const int wrow0 = q0 + 32 * w;
    // tiles this wave computes on (a causal wave stops at its diagonal)
    const int nkt_w = (wrow0 >= N) ? 0 : (CAUSAL ? min(nkt, (wrow0 + 31) / BC + 1) : nkt);

    // Copy K or V tile kt into an LDS buffer.  Each lane's byte offsets inside
    // a tile (row and swizzled chunk) are fixed for the whole kernel; the tile
    // is addressed by a buffer resource that starts at the tile and ends at
    // the end of the head, so the per-tile work is scalar and rows past the
    // end read as zero (they are masked for K and weighted by 0 for V).
    // One head's K or V is below 2^32 bytes (checked by the host).
    uint32_t k_dma[SPW], v_dma[SPW];
#pragma unroll
    for (int i = 0; i < SPW; ++i) {
        const int row = (w * SPW + i) * RPS + lane / CPR;
        const int pc = lane % CPR;
        k_dma[i] = (uint32_t)(row * ROWB + 16 * (pc ^ k_swz<D>(row)));
        v_dma[i] = (uint32_t)(row * ROWB + 16 * (pc ^ v_swz<D>(row)));
    }
    auto issue = [&](int kt, char* dst, bool is_v) __attribute__((always_inline)) {
        const __bf16* base = (is_v ? Vh : Kh) + (size_t)kt * BC * D;
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(base, (uint32_t)(N - kt * BC) * ROWB);
#pragma unroll
        for (int i = 0; i < SPW; ++i) b2lds16(rs, is_v ? v_dma[i] : k_dma[i], dst + (w * SPW + i) * 1024);
    };

    // Per-lane LDS byte offsets, fixed for the whole kernel (the swizzles only
    // depend on the low bits of the row, which the tile loops do not change).
    //  K: A operand of S^T, row 32*kb + l32, logical chunk 2*ks + g.
    int k_off[D / 16];
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) k_off[ks] = l32 * ROWB + 16 * ((2 * ks + g) ^ k_swz<D>(l32));
    //  V: transposed read of rows 16*ks + 8*h + vr, columns 32*mb + vc .. +3.
    const int vr = 4 * g + ((lane & 15) >> 2);
    const int vc = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    const int vsw = v_swz<D>(vr) >> 2;   // XOR on the chunk bits above the 4-chunk group
    int v_off[D / 32];
#pragma unroll
    for (int mb = 0; mb < D / 32; ++mb) v_off[mb] = vr * ROWB + 16 * (4 * (mb ^ vsw) + (vc >> 3)) + 2 * (vc & 7);

    // key kv0 + 32*kb + 8*(r/4) + 4*g + r%4 is hidden iff 32*kb + 8*(r/4) + r%4 > lim
    const int last_visible = CAUSAL ? min(qrow, N - 1) : N - 1;

    f32x16 oacc[D / 32];
#pragma unroll
    for (int mb = 0; mb < D / 32; ++mb) oacc[mb] = zero16();
    float m_ref = -INFINITY;   // reference max (log2 units) the exponentials use
    float l_run = 0.f;         // this lane's share of the running sum

    auto qk = [&](const char* Ks, f32x16* s) __attribute__((always_inline)) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) s[kb] = zero16();
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks)
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                const bf16x8 a = *reinterpret_cast<const bf16x8*>(Ks + 32 * kb * ROWB + k_off[ks]);
                s[kb] = mfma_bf16(a, qf[ks], s[kb]);
            }
        // Keep QK_AHEAD K-operand reads in flight ahead of the MFMAs.
        __builtin_amdgcn_sched_group_barrier(0x100, QK_AHEAD, 0);            // LDS reads
#pragma unroll
        for (int i = 0; i < NKB * D / 16 - QK_AHEAD; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);               // MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, QK_AHEAD, 0);
    };
    // mask tile kt of S (branch-free; lim is large when nothing is hidden)
    auto mask = [&](int kt, f32x16* s) __attribute__((always_inline)) {
        const int lim = last_visible - kt * BC - 4 * g;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                s[kb][r] = (32 * kb + 8 * (r >> 2) + (r & 3) > lim) ? -INFINITY : s[kb][r];
    };
    // P = 2^(c*S - m_ref) (bf16) laid out as the B operand of O^T += V^T P^T;
    // returns this lane's sum of the same bf16-rounded values the PV product
    // uses (dot2 against 1).
    auto probs = [&](const f32x16* s, bf16x8* pb) __attribute__((always_inline)) -> float {
        const float m_use = (m_ref == -INFINITY) ? 0.f : m_ref;
        float psum[2] = {0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                uint32_t pk[4];
#pragma unroll
                for (int j = 0; j < 8; j += 2) {
                    const float p0 = exp2_fast(fmaf(s[kb][8 * h + j], c, -m_use));
                    const float p1 = exp2_fast(fmaf(s[kb][8 * h + j + 1], c, -m_use));
                    pk[j / 2] = pack_bf16x2(p0, p1);
                    psum[h] = sum_bf16x2(pk[j / 2], psum[h]);
                }
                pb[2 * kb + h] = as_bf16x8(make_uint4(pk[0], pk[1], pk[2], pk[3]));
            }
        return psum[0] + psum[1];
    };
    // Lazy rescaling without a per-tile max.  The tile's exponentials are
    // first taken against the current reference m_ref.  Every probability is
    // non-negative, so a lane sum of at most P_MAX bounds each of them by
    // P_MAX, and the tile is kept.  Otherwise (some value overflowed or grew
    // large, or the row has no reference yet) the tile's row max is taken,
    // the reference is raised to it if larger -- O and l are rescaled by the
    // same factor, so numerator and denominator stay consistent -- and the
    // exponentials are recomputed.
    auto softmax = [&](const f32x16* s, bf16x8* pb) __attribute__((always_inline)) {
        float ps = probs(s, pb);
        if (__any(!(ps <= P_MAX) || m_ref == -INFINITY)) {
            float mx = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
            mx = xor32_max(mx) * c;
            if (mx > m_ref) {
                const float alpha = exp2_fast(m_ref - mx);   // 0 while the reference is -inf
                m_ref = mx;
                l_run *= alpha;
#pragma unroll
                for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) oacc[mb][r] *= alpha;
            }
            ps = probs(s, pb);
        }
        l_run += ps;
    };
    // O^T += V^T P^T ; V^T operand read transposed from the row-major tile
    auto pv = [&](const char* Vs, const bf16x8* pb) __attribute__((always_inline)) {
#pragma unroll
        for (int ks = 0; ks < BC / 16; ++ks)
#pragma unroll
            for (int mb = 0; mb < D / 32; ++mb) {
                const uint2 lo = lds_read_tr16x4(Vs + (16 * ks) * ROWB + v_off[mb]);
                const uint2 hi = lds_read_tr16x4(Vs + (16 * ks + 8) * ROWB + v_off[mb]);
                const bf16x8 a = as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
                oacc[mb] = mfma_bf16(a, pb[ks], oacc[mb]);
            }
        // Keep the V^T reads of PV_AHEAD products in flight ahead of the MFMAs.
        constexpr int n = (BC / 16) * (D / 32);
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * PV_AHEAD, 0);       // LDS reads
#pragma unroll
        for (int i = 0; i < n - PV_AHEAD; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);               // MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, PV_AHEAD, 0);
    };

    // One tile: wait for its copies, start the next tile's copies into the
    // other buffer pair, then S = K Q^T, mask, softmax and O += V^T P.
    auto step = [&](int kt, const char* kc, const char* vcb, char* kn, char* vn) __attribute__((always_inline)) {
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (kt + 1 < nkt) {
            issue(kt + 1, kn, false);
            issue(kt + 1, vn, true);
        }
        if (kt >= nkt_w) return;
        f32x16 s[NKB];
        qk(kc, s);
        if ((kt * BC + BC > N) || (CAUSAL && kt * BC + BC - 1 > wrow0)) mask(kt, s);
        bf16x8 pb[BC / 16];
        softmax(s, pb);
        pv(vcb, pb);
    };
    if (nkt > 0) {
        issue(0, kb0, false);
        issue(0, vb0, true);
    }
    for (int kt = 0; kt < nkt; kt += 2) {
        step(kt, kb0, vb0, kb1, vb1);
        if (kt + 1 < nkt) step(kt + 1, kb1, vb1, kb0, vb0);
    }

    const float l_tot = xor32_sum(l_run);
    const float inv = (l_tot > 0.f) ? 1.f / l_tot : 0.f;
    if constexpr (OUT_BF16 && D <= 128) {
        // Each lane holds 8 bytes of 16 rows of O.  Stored directly, every
        // store instruction would write 16 bytes into each of 32 rows; the
        // rows go through the (now free) tile buffers instead -- wave w uses
        // one of them, chunks XOR-permuted by the row -- and each store then
        // writes whole rows.  (At d = 256 the extra registers would spill
        // under the two-waves-per-SIMD budget, so it stores directly.)
        constexpr int CH = D / 8;                  // 16-byte chunks per row
        static_assert(32 * ROWB <= TILEB, "a wave's O rows fit one tile buffer");
        __syncthreads();                           // every wave is done with the tiles
        char* sb = w == 0 ? kb0 : w == 1 ? kb1 : w == 2 ? vb0 : vb1;
#pragma unroll
        for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
            for (int rb = 0; rb < 4; ++rb) {
                const int off = l32 * ROWB + 16 * ((4 * mb + rb) ^ (l32 % CH)) + 8 * g;
                *reinterpret_cast<uint2*>(sb + off) =
                    make_uint2(pack_bf16x2(oacc[mb][4 * rb + 0] * inv, oacc[mb][4 * rb + 1] * inv),
                               pack_bf16x2(oacc[mb][4 * rb + 2] * inv, oacc[mb][4 * rb + 3] * inv));
            }
        constexpr int RPP = 64 / CH < 1 ? 1 : 64 / CH;   // rows per pass
        constexpr int LPR = CH < 64 ? CH : 64;           // lanes per row in a pass
#pragma unroll
        for (int p = 0; p < 32 / RPP; ++p)
#pragma unroll
            for (int c0 = 0; c0 < CH; c0 += LPR) {
                const int r = RPP * p + lane / LPR, ch = c0 + lane % LPR;
                const uint4 v4 = *reinterpret_cast<const uint4*>(sb + r * ROWB + 16 * (ch ^ (r % CH)));
                if (wrow0 + r < N)
                    *reinterpret_cast<uint4*>(static_cast<__bf16*>(O) + (size_t)bh * N * D +
                                              (size_t)(wrow0 + r) * D + 8 * ch) = v4;
            }
    } else if (qrow < N) {
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
    }
    if (qrow < N && g == 0)
        LSE[(size_t)bh * N + qrow] = (l_tot > 0.f) ? m_ref * kLn2 + __logf(l_tot) : -INFINITY;
    if constexpr (CLOCK) {
        if (tid == 0) {
            clk[2 * blockIdx.x] = __builtin_amdgcn_s_memtime() - clk_t0;
            clk[2 * blockIdx.x + 1] = __builtin_amdgcn_s_memrealtime() - clk_r0;
        }
    }
}

}  // namespace

}  // namespace fa
