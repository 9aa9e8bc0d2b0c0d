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
// Two launches on the caller's stream (three with the grouped split):
//   1. bwd_dq:    one workgroup per tile of 128 query rows, streaming the K/V
//                 tiles of its head like the forward pass: it recomputes S, P
//                 and dP, forms dS and accumulates dQ^T = K^T dS^T in
//                 registers.  Each lane holds half of its query row's dO, so
//                 it also forms that row's D = rowsum(dO * O) in fp32 (one
//                 exchange with lane ^ 32) and writes D and the LSE in base-2
//                 units (LSE log2 e) to the workspace for the next kernel.
//                 Recomputing S and dP a second time costs three more matrix
//                 products than accumulating dQ with atomics from the key-tile
//                 kernel, but those atomics measured slower than the
//                 products, and this way dQ needs no fp32 accumulator, no
//                 extra pass and is deterministic.
//   2. bwd_dkdv:  one workgroup per tile of BC = 128 keys of one K/V head (4
//                 waves, 32 keys each), walking the query tiles (BR = 64 rows)
//                 that can see its keys -- for each of the H/Hkv query heads
//                 sharing that K/V head, so a shared head's gradient is summed
//                 in registers.  K and V of the tile stay in registers; Q, dO,
//                 the base-2 LSE and D of the next query tile are copied global -> LDS by
//                 buffer DMA while the current one is computed.  dK^T and dV^T
//                 accumulate in registers and are stored once, staged through
//                 the free tile buffers so that each store writes whole rows.
//                 With grouped heads and a grid of few workgroups the causal
//                 imbalance between key tiles would decide the run time; then
//                 each group of s query heads (s dividing H/Hkv, chosen to
//                 give just enough workgroups) gets workgroups of its own,
//                 which store fp32 partial dK^T / dV^T rows, and bwd_kv_reduce
//                 sums them over the groups in order (a third launch).
//
// Layout trick (as in the forward): with queries as MFMA rows and keys as
// columns, each lane holds one key and 16 queries, and those registers are
// directly the K-slot-ordered B operands of dV^T = dO^T P and dK^T = Q^T dS;
// with keys as rows and queries as columns (dQ kernel) each lane holds one
// query and 16 keys, the B operand of dQ^T = K^T dS^T.  The transposed A
// operands (Q^T, dO^T, K^T) are read with the transposing LDS read in the
// matching order.
#include <type_traits>

#include "fa_common.hpp"
#include "fa_internal.hpp"

namespace fa {

namespace {

// Query rows per inner step of the dK/dV kernel: 64 (two 32-row halves whose
// products and exponentials are interleaved) for d <= 128.  At d = 256 the
// wave's K and V (128 VGPRs) and its dK^T/dV^T accumulators (256 registers)
// leave room for one 32-row block only.
template <int D>
constexpr int bwd_br() { return D == 256 ? 32 : 64; }
constexpr int BWD_BC = kBwdKeyTile;   // keys per workgroup (4 waves x 32)
constexpr int BWD_THREADS = 256;

// ---------------------------------------------------------------------------
// dK/dV kernel
// ---------------------------------------------------------------------------
// Q and dO tiles live in LDS row-major (2*D bytes per row, no padding),
// filled by direct global -> LDS copies.  Each is read two ways: 16-byte
// chunks by 32 consecutive rows (A operands of S = Q K^T and dP = dO V^T) and
// with the transposing 8-byte read (Q^T and dO^T operands); rt_swz keeps both
// patterns free of bank conflicts.
// Ask the scheduler to interleave the current region as n groups of
// (rd LDS reads, 1 MFMA, va VALU ops), so that vector work issues while the
// matrix core is busy with the same wave's products.
#define FA_INTERLEAVE(n, rd, va)                                   \
    do {                                                           \
        _Pragma("unroll") for (int _i = 0; _i < (n); ++_i) {       \
            __builtin_amdgcn_sched_group_barrier(0x100, (rd), 0);  \
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);     \
            __builtin_amdgcn_sched_group_barrier(0x002, (va), 0);  \
        }                                                          \
    } while (0)

// s_waitcnt with only vmcnt constrained (expcnt / lgkmcnt left at their max).
#define FA_WAIT_VMCNT(n) \
    __builtin_amdgcn_s_waitcnt((((n) & 15) | (((n) >> 4) << 14)) | (7 << 4) | (15 << 8))
#define FA_WAIT_LGKM0() __builtin_amdgcn_s_waitcnt((15) | (3 << 14) | (7 << 4))

// SPLIT: one workgroup per (group of HPG query heads, key tile) instead of per
// (K/V head, key tile); the group's unscaled dK^T / dV^T rows go to the fp32
// partial buffers pdk / pdv ([B*H/HPG, N, D]) and bwd_kv_reduce_kernel sums
// them.
template <int D, bool CAUSAL, bool SPLIT>
__global__ void __launch_bounds__(BWD_THREADS)
bwd_dkdv_kernel(const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
                const __bf16* __restrict__ dO, const float* __restrict__ LSE2 /* LSE log2 e */,
                const float* __restrict__ delta, __bf16* __restrict__ dK,
                __bf16* __restrict__ dV, float* __restrict__ pdk, float* __restrict__ pdv,
                int BHkv, int G, int HPG, int N, float c /* scale*log2e */, float scale) {
    constexpr int BR = bwd_br<D>(), BC = BWD_BC;
    constexpr int ROWB = 2 * D;                  // bytes per row of a Q/dO/K tile
    constexpr int CPR = D / 8;
    constexpr int QTB = BR * ROWB;               // bytes of a Q (or dO) tile
    constexpr int RPS = 1024 / ROWB;             // rows per 1 KiB copy segment
    constexpr int QSPW = QTB / 1024 / 4;         // Q segments per wave
    constexpr int NQB = BR / 32;
    static_assert(QSPW >= 1, "tile shapes");

    // Two buffers, each holding a query tile's Q, dO, LSE and D.  They are
    // separate LDS objects, so the compiler can tell that the copies into one
    // do not alias the reads of the other and need not wait for them.
    constexpr int BUFB = 2 * QTB + 2 * BR * 4;
    __shared__ __attribute__((aligned(1024))) char buf0[BUFB];
    __shared__ __attribute__((aligned(1024))) char buf1[BUFB];
    static_assert(BR == 64 || BR == 32, "one or two 32-row blocks per query tile; one wave copies a row statistic");

    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const int l32 = lane & 31, g = lane >> 5;

    // One workgroup per (K/V head, key tile); heavy tiles first: key tile 0
    // sees every query tile.  The G query heads sharing this K/V head are
    // visited in turn, so dK and dV sum their contributions in registers.
    // SPLIT: one workgroup per (group of HPG query heads, key tile); the G/HPG
    // groups of a K/V head are B*Hkv block ids apart.  Its fp32 partial rows go
    // to partial block `part` = K/V head * (G/HPG) + group.
    const int NHG = SPLIT ? HPG : G;              // query heads this workgroup visits
    int kvh, kt, head0, part = 0;                 // K/V head, key tile, first query head
    if constexpr (SPLIT) {
        const int NGR = G / HPG, BG = BHkv * NGR, j = blockIdx.x % BG;
        kt = blockIdx.x / BG;
        kvh = j % BHkv;
        const int grp = j / BHkv;
        head0 = kvh * G + grp * HPG;
        part = kvh * NGR + grp;
    } else {
        kvh = blockIdx.x % BHkv;
        kt = blockIdx.x / BHkv;
        head0 = kvh * G;
    }
    const int k0 = kt * BC;
    const size_t kvoff = (size_t)kvh * (size_t)N * D;
    const __bf16* Kh = K + kvoff;
    const __bf16* Vh = V + kvoff;

    // Copy rows [r0, r0 + BR) of one head's [N, D] tensor (below 2^32 bytes,
    // checked by the host) into an LDS tile.  Each lane's byte offsets inside
    // the tile depend only on the lane; the tile is addressed by a buffer resource that
    // starts at row r0 and ends at the end of the head, so rows past the end
    // read as zero (they are masked).
    auto issue = [&](const __bf16* head, int r0, char* dst) __attribute__((always_inline)) {
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(head + (size_t)r0 * D, (uint32_t)(N - r0) * ROWB);
#pragma unroll
        for (int i = 0; i < QSPW; ++i) {
            const int row = (w * QSPW + i) * RPS + lane / CPR;
            b2lds16(rs, (uint32_t)(row * ROWB + 16 * ((lane % CPR) ^ rt_swz<D>(row))), dst + (w * QSPW + i) * 1024);
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
    // The swizzle only permutes the low 4 bits of the chunk index, so at d = 256
    // chunks 16..31 sit 256 bytes after chunks 0..15: eight offsets serve all
    // K-steps (register pressure).
    constexpr int NRO = D / 16 > 8 ? 8 : D / 16;
    int rd_off_[NRO];
#pragma unroll
    for (int ks = 0; ks < NRO; ++ks) rd_off_[ks] = l32 * ROWB + 16 * ((2 * ks + g) ^ rt_swz<D>(l32));
    auto rd_off = [&](int ks) __attribute__((always_inline)) -> int { return rd_off_[ks % NRO] + 256 * (ks / NRO); };
    // Transposed reads: the 16-lane group of this lane reads rows r..r+3 and
    // columns 32*mb + ct .. +15, lane (rt, ct): row r + rt, 4 columns at ct.
    // Row offsets that are multiples of 16 leave the swizzle unchanged, so the
    // Q^T / dO^T rows 16*ks + 4*g + 8*h + rt need one per-lane offset per
    // (h, mb): qt_off[h][mb] + 16*ks*ROWB.
    const int rt = (lane & 15) >> 2;
    const int ct = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    auto tr_off = [&](int row, int col) __attribute__((always_inline)) -> int {
        return row * ROWB + 16 * ((col >> 3) ^ rt_swz<D>(row)) + 2 * (col & 7);
    };
    constexpr int NTO = D / 32 > 4 ? 4 : D / 32;   // as above: columns 128.. sit 256 bytes on
    int qt_off_[2][NTO];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int mb = 0; mb < NTO; ++mb) qt_off_[h][mb] = tr_off(4 * g + 8 * h + rt, 32 * mb + ct);
    auto qt_off = [&](int h, int mb) __attribute__((always_inline)) -> int {
        return qt_off_[h][mb % NTO] + 256 * (mb / NTO);
    };

    f32x16 dvt[D / 32], dkt[D / 32];
#pragma unroll
    for (int mb = 0; mb < D / 32; ++mb) {
        dvt[mb] = zero16();
        dkt[mb] = zero16();
    }

    const int nqt = (N + BR - 1) / BR;
    const int qt_begin = CAUSAL ? (k0 / BR) : 0;

    // Work items: (query head head0 + r, query tile qt) for r < NHG and
    // qt = qt_begin..nqt-1, flattened to it = r * nq + (qt - qt_begin).
    const int nq = nqt - qt_begin;
    const int n_items = NHG * nq;

    // buffer layout: Q tile | dO tile | LSE[BR] | D[BR].  LSE (wave 0) and D
    // (wave 1) are one row per lane; rows past the end read as zero (and are
    // masked).  Work item (r, q): query head r of the group, query tile
    // qt_begin + q.
    auto fill = [&](int r, int q, char* b) __attribute__((always_inline)) {
        const size_t qh = (size_t)head0 + r;
        const int r0 = (qt_begin + q) * BR;
        issue(Q + qh * N * D, r0, b);
        issue(dO + qh * N * D, r0, b + QTB);
        const uint32_t nb = (uint32_t)(N - r0) * 4;
        if (w == 0 && lane < BR)
            b2lds4(make_rsrc(LSE2 + qh * N + r0, nb), 4 * lane, reinterpret_cast<float*>(b + 2 * QTB));
        if (w == 1 && lane < BR)
            b2lds4(make_rsrc(delta + qh * N + r0, nb), 4 * lane, reinterpret_cast<float*>(b + 2 * QTB + 4 * BR));
    };
    // running (r, q) of the item being computed and of the next one to copy,
    // in the order it = r * nq + q
    int cur_q = 0, nxt_r = 0, nxt_q = 0;
    auto advance = [&](int& r, int& q) __attribute__((always_inline)) {
        if (++q == nq) {
            q = 0;
            ++r;
        }
    };

    // prologue: the first work item
    if (n_items > 0) {
        fill(0, 0, buf0);
        advance(nxt_r, nxt_q);
    }
    FA_WAIT_VMCNT(0);

    auto tile = [&](int it, const char* cur, char* nxt) __attribute__((always_inline)) {
        const char* qs = cur;
        const char* os = cur + QTB;
        const float* ls = reinterpret_cast<const float*>(cur + 2 * QTB);
        const float* ds_ = reinterpret_cast<const float*>(cur + 2 * QTB + 4 * BR);
        const int q0 = (qt_begin + cur_q) * BR;
        if (++cur_q == nq) cur_q = 0;
        // copies of this tile have landed, and every wave is done with the
        // previous tile, so its buffers may be refilled
        FA_WAIT_VMCNT(0);
        __builtin_amdgcn_s_barrier();
        if (it + 1 < n_items) {
            fill(nxt_r, nxt_q, nxt);
            advance(nxt_r, nxt_q);
        }

        // a wave whose keys see none of the tile's queries has nothing to add
        const bool wave_dead = (CAUSAL && wk0 > q0 + BR - 1) || wk0 >= N;
        if (!wave_dead) {
            // LSE and D of this lane's 16 query rows per block (runs of 4);
            // at d = 256 they are read where they are used (register pressure)
            float4 lse4[NQB][4], dd4[NQB][4];
            if constexpr (D != 256) {
#pragma unroll
                for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
                    for (int rb = 0; rb < 4; ++rb) {
                        lse4[qb][rb] = *reinterpret_cast<const float4*>(ls + 32 * qb + 8 * rb + 4 * g);
                        dd4[qb][rb] = *reinterpret_cast<const float4*>(ds_ + 32 * qb + 8 * rb + 4 * g);
                    }
            }

            // The two 32-row halves of the tile are independent until they
            // meet in dV^T and dK^T, which lets one half's exponentials run in
            // the shadow of the other half's matrix products:
            //   S,dP(0) | S,dP(1) + P,dS(0) | dV,dK(0) + P,dS(1) | dV,dK(1)
            f32x16 sP[NQB], dP[NQB];
            bf16x8 pb[BR / 16], sb[BR / 16];
            auto sdp = [&](int qb) __attribute__((always_inline)) {
                sP[qb] = zero16();
                dP[qb] = zero16();
#pragma unroll
                for (int ks = 0; ks < D / 16; ++ks) {
                    const bf16x8 aq = *reinterpret_cast<const bf16x8*>(qs + 32 * qb * ROWB + rd_off(ks));
                    sP[qb] = mfma_bf16(aq, kf[ks], sP[qb]);
                    const bf16x8 ad = *reinterpret_cast<const bf16x8*>(os + 32 * qb * ROWB + rd_off(ks));
                    dP[qb] = mfma_bf16(ad, vf[ks], dP[qb]);
                }
            };
            // P = 2^(c S - LSE log2 e), masked; dS = P (dP - D); both packed to
            // bf16 as the B operands of the two K-steps of this half
            auto pds = [&](int qb, auto masked, int h0 = 0, int h1 = 2) __attribute__((always_inline)) {
#pragma unroll
                for (int h = h0; h < h1; ++h) {
                    uint32_t pk[4], sk[4];
#pragma unroll
                    for (int j = 0; j < 8; j += 2) {
                        float pv[2], sv[2];
#pragma unroll
                        for (int u = 0; u < 2; ++u) {
                            const int r = 8 * h + j + u, rb = r >> 2, t = r & 3;
                            const float4 l4 = D == 256 ? *reinterpret_cast<const float4*>(ls + 32 * qb + 8 * rb + 4 * g)
                                                       : lse4[qb][rb];
                            const float4 d4 = D == 256 ? *reinterpret_cast<const float4*>(ds_ + 32 * qb + 8 * rb + 4 * g)
                                                       : dd4[qb][rb];
                            const float lv = t == 0 ? l4.x : t == 1 ? l4.y : t == 2 ? l4.z : l4.w;
                            const float dv = t == 0 ? d4.x : t == 1 ? d4.y : t == 2 ? d4.z : d4.w;
                            float p = exp2_fast(fmaf(sP[qb][r], c, -lv));
                            if (decltype(masked)::value) {
                                const int qrow = q0 + 32 * qb + 8 * rb + 4 * g + t;
                                if (!key_live || qrow >= N || (CAUSAL && key > qrow)) p = 0.f;
                            }
                            pv[u] = p;
                            sv[u] = p * (dP[qb][r] - dv);
                        }
                        pk[j / 2] = pack_bf16x2(pv[0], pv[1]);
                        sk[j / 2] = pack_bf16x2(sv[0], sv[1]);
                    }
                    pb[2 * qb + h] = as_bf16x8(make_uint4(pk[0], pk[1], pk[2], pk[3]));
                    sb[2 * qb + h] = as_bf16x8(make_uint4(sk[0], sk[1], sk[2], sk[3]));
                }
            };
            // dV^T += dO^T P ; dK^T += Q^T dS for K-step ks (queries
            // 16*ks + 4*g + {0..3, 8..11}, the C-layout order of P and dS)
            auto dvdk = [&](int ks) __attribute__((always_inline)) {
                const int rk = 16 * ks * ROWB;
#pragma unroll
                for (int mb = 0; mb < D / 32; ++mb) {
                    const uint2 dlo = lds_read_tr16x4(os + rk + qt_off(0, mb));
                    const uint2 dhi = lds_read_tr16x4(os + rk + qt_off(1, mb));
                    dvt[mb] = mfma_bf16(as_bf16x8(make_uint4(dlo.x, dlo.y, dhi.x, dhi.y)), pb[ks], dvt[mb]);
                    const uint2 qlo = lds_read_tr16x4(qs + rk + qt_off(0, mb));
                    const uint2 qhi = lds_read_tr16x4(qs + rk + qt_off(1, mb));
                    dkt[mb] = mfma_bf16(as_bf16x8(make_uint4(qlo.x, qlo.y, qhi.x, qhi.y)), sb[ks], dkt[mb]);
                }
            };
            auto pipeline = [&](auto masked) __attribute__((always_inline)) {
                if constexpr (NQB == 2) {
                    sdp(0);
                    __builtin_amdgcn_sched_barrier(0);
                    sdp(1);
                    pds(0, masked);
                    FA_INTERLEAVE(2 * D / 16, 2, 4);
                    __builtin_amdgcn_sched_barrier(0);
                    dvdk(0);
                    dvdk(1);
                    pds(1, masked);
                    FA_INTERLEAVE(4 * D / 32, 4, 4);
                    __builtin_amdgcn_sched_barrier(0);
                    dvdk(2);
                    dvdk(3);
                } else {
                    // one 32-row block: S, dP | P, dS of rows 0..15 | dV, dK
                    // of K-step 0 beside P, dS of rows 16..31 | dV, dK of
                    // K-step 1
                    sdp(0);
                    pds(0, masked, 0, 1);
                    __builtin_amdgcn_sched_barrier(0);
                    dvdk(0);
                    pds(0, masked, 1, 2);
                    FA_INTERLEAVE(2 * D / 32, 4, 4);
                    __builtin_amdgcn_sched_barrier(0);
                    dvdk(1);
                }
            };
            // Causal: the unmasked copy serves every tile off the diagonal.
            // Without a causal mask no tile needs one: query rows past N
            // read as zero (Q, dO, LSE and D), so P = 1 there while dO and
            // dS vanish, and they add nothing to dK or dV; keys past N have
            // zero K and V, and only their own dK/dV columns (never stored)
            // see them.
            if constexpr (D == 256) {
                // one copy of the body, the masked one: at d = 256 the causal
                // kernel with both copies spills, and the unmasked body alone
                // still spills a few registers
                pipeline(std::true_type{});
            } else if constexpr (CAUSAL) {
                const bool need_mask = (k0 + BC > N) || (q0 + BR > N) || (wk0 + 31 > q0);
                if (need_mask)
                    pipeline(std::true_type{});
                else
                    pipeline(std::false_type{});
            } else {
                pipeline(std::false_type{});
            }
        }
    };

    for (int it = 0; it < n_items; it += 2) {
        tile(it, buf0, buf1);
        if (it + 1 < n_items) tile(it + 1, buf1, buf0);
    }

    // dV = (dV^T)^T, dK = scale (dK^T)^T: lane holds key `key`, dims in runs of 4
    if constexpr (D == 256) {
        // d = 256: 128 rows of 512 bytes per tensor do not fit the two tile
        // buffers, so every lane writes its 16-byte runs directly (the
        // epilogue is small against the query loop at these sizes)
        if (key_live) {
#pragma unroll
            for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
                for (int rb = 0; rb < 4; ++rb) {
                    const int d0 = 32 * mb + 8 * rb + 4 * g;
                    if constexpr (SPLIT) {
                        const size_t o = ((size_t)part * N + key) * D + d0;
                        *reinterpret_cast<float4*>(pdv + o) =
                            make_float4(dvt[mb][4 * rb], dvt[mb][4 * rb + 1], dvt[mb][4 * rb + 2], dvt[mb][4 * rb + 3]);
                        *reinterpret_cast<float4*>(pdk + o) =
                            make_float4(dkt[mb][4 * rb], dkt[mb][4 * rb + 1], dkt[mb][4 * rb + 2], dkt[mb][4 * rb + 3]);
                    } else {
                        const size_t o = kvoff + (size_t)key * D + d0;
                        *reinterpret_cast<uint2*>(dV + o) =
                            make_uint2(pack_bf16x2(dvt[mb][4 * rb], dvt[mb][4 * rb + 1]),
                                       pack_bf16x2(dvt[mb][4 * rb + 2], dvt[mb][4 * rb + 3]));
                        *reinterpret_cast<uint2*>(dK + o) =
                            make_uint2(pack_bf16x2(scale * dkt[mb][4 * rb], scale * dkt[mb][4 * rb + 1]),
                                       pack_bf16x2(scale * dkt[mb][4 * rb + 2], scale * dkt[mb][4 * rb + 3]));
                    }
                }
        }
    } else if constexpr (SPLIT) {
        // The fp32 partial rows go through the free tile buffers too (waves
        // 0 and 1 in buf0, 2 and 3 in buf1; dV, then dK in the same rows),
        // so that each store writes whole rows rather than 16 bytes into each
        // of 32 rows.
        constexpr int RB = 4 * D;                  // bytes per fp32 row
        constexpr int CHF = D / 4;                 // 16-byte chunks per row
        constexpr int RPPF = 64 / CHF;             // rows per pass, one chunk per lane
        static_assert(64 * RB <= BUFB, "two waves' fp32 rows fit a tile buffer");
        __syncthreads();                           // every wave is done with the tiles
        char* wb = (w < 2 ? buf0 : buf1) + (w & 1) * 32 * RB;
        auto stagef = [&](const f32x16* acc, float* dst) __attribute__((always_inline)) {
#pragma unroll
            for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
                for (int rb = 0; rb < 4; ++rb)
                    *reinterpret_cast<float4*>(wb + l32 * RB + 16 * ((8 * mb + 2 * rb + g) ^ (l32 % CHF))) =
                        make_float4(acc[mb][4 * rb], acc[mb][4 * rb + 1], acc[mb][4 * rb + 2], acc[mb][4 * rb + 3]);
#pragma unroll
            for (int p = 0; p < 32 / RPPF; ++p) {
                const int r = RPPF * p + lane / CHF, ch = lane % CHF;
                const float4 v = *reinterpret_cast<const float4*>(wb + r * RB + 16 * (ch ^ (r % CHF)));
                if (wk0 + r < N) *reinterpret_cast<float4*>(dst + ((size_t)part * N + wk0 + r) * D + 4 * ch) = v;
            }
        };
        stagef(dvt, pdv);
        stagef(dkt, pdk);
    }
    if constexpr (!SPLIT && D != 256) {
        // Each lane holds 8 bytes of 16 rows; stored directly, every store
        // instruction would write 16 bytes into each of 32 rows, which held
        // the waves for microseconds at the end of every workgroup.  The rows
        // go through the (now free) tile buffers instead: dV in buf0, dK in
        // buf1, row 32w + l32 of the tile, 16-byte chunks XOR-permuted by the
        // row so the writes spread over the banks; then each store writes
        // whole rows.
        constexpr int CH = D / 8;                  // 16-byte chunks per row
        static_assert(128 * ROWB <= BUFB, "dK/dV staging fits a tile buffer");
        __syncthreads();                           // every wave is done with the tiles
        const int srow = 32 * w + l32;
#pragma unroll
        for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
            for (int rb = 0; rb < 4; ++rb) {
                const int off = srow * ROWB + 16 * ((4 * mb + rb) ^ (srow % CH)) + 8 * g;
                *reinterpret_cast<uint2*>(buf0 + off) =
                    make_uint2(pack_bf16x2(dvt[mb][4 * rb], dvt[mb][4 * rb + 1]),
                               pack_bf16x2(dvt[mb][4 * rb + 2], dvt[mb][4 * rb + 3]));
                *reinterpret_cast<uint2*>(buf1 + off) =
                    make_uint2(pack_bf16x2(scale * dkt[mb][4 * rb], scale * dkt[mb][4 * rb + 1]),
                               pack_bf16x2(scale * dkt[mb][4 * rb + 2], scale * dkt[mb][4 * rb + 3]));
            }
        // this wave's 32 rows back, 64 / CH rows per pass, one chunk per lane
        constexpr int RPP = 64 / CH;
#pragma unroll
        for (int p = 0; p < 32 / RPP; ++p) {
            const int r = 32 * w + RPP * p + lane / CH, ch = lane % CH;
            const int off = r * ROWB + 16 * (ch ^ (r % CH));
            const uint4 v4 = *reinterpret_cast<const uint4*>(buf0 + off);
            const uint4 k4 = *reinterpret_cast<const uint4*>(buf1 + off);
            if (k0 + r < N) {
                const size_t g0 = kvoff + (size_t)(k0 + r) * D + 8 * ch;
                *reinterpret_cast<uint4*>(dV + g0) = v4;
                *reinterpret_cast<uint4*>(dK + g0) = k4;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Sum of the split dK/dV partials over the NGR head groups of each K/V head,
// in group order (deterministic); dK is scaled here.  Eight elements per
// thread.
// ---------------------------------------------------------------------------
template <int D>
__global__ void __launch_bounds__(256)
bwd_kv_reduce_kernel(const float* __restrict__ pdk, const float* __restrict__ pdv, __bf16* __restrict__ dK,
                     __bf16* __restrict__ dV, long long n8, int NGR, int N, float scale) {
    const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
    if (i >= n8) return;
    const long long e = 8 * i;                          // element of [B*Hkv, N, D]
    const long long per_head = (long long)N * D;
    const long long kvh = e / per_head, rem = e - kvh * per_head;
    float sk[8] = {}, sv[8] = {};
    for (int r = 0; r < NGR; ++r) {
        const size_t src = (size_t)((kvh * NGR + r) * per_head + rem);
        const float4 k0 = *reinterpret_cast<const float4*>(pdk + src);
        const float4 k1 = *reinterpret_cast<const float4*>(pdk + src + 4);
        const float4 v0 = *reinterpret_cast<const float4*>(pdv + src);
        const float4 v1 = *reinterpret_cast<const float4*>(pdv + src + 4);
        sk[0] += k0.x; sk[1] += k0.y; sk[2] += k0.z; sk[3] += k0.w;
        sk[4] += k1.x; sk[5] += k1.y; sk[6] += k1.z; sk[7] += k1.w;
        sv[0] += v0.x; sv[1] += v0.y; sv[2] += v0.z; sv[3] += v0.w;
        sv[4] += v1.x; sv[5] += v1.y; sv[6] += v1.z; sv[7] += v1.w;
    }
    *reinterpret_cast<uint4*>(dK + e) =
        make_uint4(pack_bf16x2(scale * sk[0], scale * sk[1]), pack_bf16x2(scale * sk[2], scale * sk[3]),
                   pack_bf16x2(scale * sk[4], scale * sk[5]), pack_bf16x2(scale * sk[6], scale * sk[7]));
    *reinterpret_cast<uint4*>(dV + e) = make_uint4(pack_bf16x2(sv[0], sv[1]), pack_bf16x2(sv[2], sv[3]),
                                                   pack_bf16x2(sv[4], sv[5]), pack_bf16x2(sv[6], sv[7]));
}

// ---------------------------------------------------------------------------
// dQ kernel: query-tile outer, K/V tiles streamed through LDS; also forms D
// and the base-2 LSE for the dK/dV kernel.
// ---------------------------------------------------------------------------
constexpr int DQ_BR = 128;       // query rows per workgroup (4 waves x 32)
// keys per K/V tile: 64, or 32 at d = 256 (as in the forward), where Q^T and
// dO^T (128 VGPRs) and the dQ^T accumulator (128) already fill one wave's
// budget at two waves per SIMD; d = 256 runs one wave per SIMD
template <int D>
constexpr int dq_bc() { return D == 256 ? 32 : 64; }

// instruction schedule of the dQ tile loop (measured best on MI355X)
constexpr int DQ_AHEAD = 2;         // K^T operands read ahead of the dQ MFMAs
constexpr int DQ_VALU_FIRST = 40;   // dS work placed before the first dQ MFMA
constexpr int DQ_VALU_EACH = 8;     // and between the following ones

template <int D, bool CAUSAL>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(D == 256 ? 1 : 2)))
bwd_dq_kernel(const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
              const __bf16* __restrict__ dO, const void* __restrict__ O, int o_bf16, const float* __restrict__ LSE,
              float* __restrict__ delta, float* __restrict__ LSE2, __bf16* __restrict__ dQ, int BH, int G, int N, int nqt, float c /* scale*log2e */, float scale) {
    constexpr int BR = DQ_BR, BC = dq_bc<D>();
    constexpr int ROWB = 2 * D;
    constexpr int CPR = D / 8;
    constexpr int TILEB = BC * ROWB;
    constexpr int RPS = 1024 / ROWB;
    constexpr int SPW = TILEB / 1024 / 4;
    constexpr int NKB = BC / 32;
    static_assert(SPW >= 1, "tile too small for four waves");

    // two buffer pairs (K tile, V tile), separate LDS objects (see the forward)
    __shared__ __attribute__((aligned(1024))) char kb0[TILEB];
    __shared__ __attribute__((aligned(1024))) char kb1[TILEB];
    __shared__ __attribute__((aligned(1024))) char vb0[TILEB];
    __shared__ __attribute__((aligned(1024))) char vb1[TILEB];

    const int tid = threadIdx.x;
    const int lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, g = lane >> 5;

    // heavy (late) query tiles first; within one sweep over the heads the G
    // query heads of a K/V head are BH / G blocks apart (same XCD when that is
    // a multiple of 8, as in the forward's block order)
    const int j = blockIdx.x % BH, NG = BH / G;
    const int bh = (j % NG) * G + j / NG;
    const int qt = CAUSAL ? (nqt - 1 - blockIdx.x / BH) : (blockIdx.x / BH);
    const int q0 = qt * BR;
    const size_t hoff = (size_t)bh * (size_t)N * D;
    const size_t kvoff = (size_t)(bh / G) * (size_t)N * D;
    const __bf16* Qh = Q + hoff;
    const __bf16* Kh = K + kvoff;
    const __bf16* Vh = V + kvoff;
    const __bf16* dOh = dO + hoff;

    // Q^T and dO^T fragments: B operands of S^T = K Q^T and dP^T = V dO^T
    const int wrow0 = q0 + 32 * w;
    const int qrow = wrow0 + l32;
    const bool row_live = qrow < N;
    bf16x8 qf[D / 16], df[D / 16];
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
        uint4 uq = make_uint4(0, 0, 0, 0), ud = uq;
        if (row_live) {
            uq = *reinterpret_cast<const uint4*>(Qh + (size_t)qrow * D + 16 * ks + 8 * g);
            ud = *reinterpret_cast<const uint4*>(dOh + (size_t)qrow * D + 16 * ks + 8 * g);
        }
        qf[ks] = as_bf16x8(uq);
        df[ks] = as_bf16x8(ud);
    }
    // D = rowsum(dO * O) of this lane's row: the lane holds chunks 16*ks + 8*g
    // of dO, lane ^ 32 the other half.  With the base-2 LSE it goes to the
    // workspace for the dK/dV kernel.  Rows past the end get LSE = +inf (P = 0).
    float dpart = 0.f;
    if (row_live) {
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
            const size_t oe = hoff + (size_t)qrow * D + 16 * ks + 8 * g;
            float ov[8];
            if (o_bf16) {
                const uint4 ou = *reinterpret_cast<const uint4*>(static_cast<const __bf16*>(O) + oe);
                const uint32_t* op = reinterpret_cast<const uint32_t*>(&ou);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    ov[2 * j] = bf16_lo(op[j]);
                    ov[2 * j + 1] = bf16_hi(op[j]);
                }
            } else {
                const float4 a = *reinterpret_cast<const float4*>(static_cast<const float*>(O) + oe);
                const float4 b = *reinterpret_cast<const float4*>(static_cast<const float*>(O) + oe + 4);
                ov[0] = a.x; ov[1] = a.y; ov[2] = a.z; ov[3] = a.w;
                ov[4] = b.x; ov[5] = b.y; ov[6] = b.z; ov[7] = b.w;
            }
            const uint4 du = __builtin_bit_cast(uint4, df[ks]);
            const uint32_t* dp = reinterpret_cast<const uint32_t*>(&du);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                dpart = fmaf(bf16_lo(dp[j]), ov[2 * j], dpart);
                dpart = fmaf(bf16_hi(dp[j]), ov[2 * j + 1], dpart);
            }
        }
    }
    const float dd = dpart + __shfl_xor(dpart, 32);
    const float lse2 = row_live ? LSE[(size_t)bh * N + qrow] * kLog2e : INFINITY;
    if (row_live && g == 0) {
        delta[(size_t)bh * N + qrow] = dd;
        LSE2[(size_t)bh * N + qrow] = lse2;
    }

    const int kv_end = CAUSAL ? min(N, q0 + BR) : N;
    const int nkt = (kv_end + BC - 1) / BC;
    const int nkt_w = (wrow0 >= N) ? 0 : (CAUSAL ? min(nkt, (wrow0 + 31) / BC + 1) : nkt);

    // K is read both ways (rows for S^T, transposed for K^T): rt_swz.
    // V is only read by rows (dP^T = V dO^T): k_swz.  Per-lane offsets inside
    // a tile are fixed; each tile is addressed by a buffer resource from its
    // first row to the end of the head, so rows past the end read as zero
    // (masked).
    uint32_t k_dma[SPW], v_dma[SPW];
#pragma unroll
    for (int i = 0; i < SPW; ++i) {
        const int row = (w * SPW + i) * RPS + lane / CPR;
        const int pc = lane % CPR;
        k_dma[i] = (uint32_t)(row * ROWB + 16 * (pc ^ rt_swz<D>(row)));
        v_dma[i] = (uint32_t)(row * ROWB + 16 * (pc ^ k_swz<D>(row)));
    }
    auto issue = [&](int kt, char* kdst, char* vdst) __attribute__((always_inline)) {
        const uint32_t nb = (uint32_t)(N - kt * BC) * ROWB;
        const __amdgpu_buffer_rsrc_t k_rs = make_rsrc(Kh + (size_t)kt * BC * D, nb);
        const __amdgpu_buffer_rsrc_t v_rs = make_rsrc(Vh + (size_t)kt * BC * D, nb);
#pragma unroll
        for (int i = 0; i < SPW; ++i) {
            b2lds16(k_rs, k_dma[i], kdst + (w * SPW + i) * 1024);
            b2lds16(v_rs, v_dma[i], vdst + (w * SPW + i) * 1024);
        }
    };

    int ko[D / 16], vo[D / 16];
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
        ko[ks] = l32 * ROWB + 16 * ((2 * ks + g) ^ rt_swz<D>(l32));
        vo[ks] = l32 * ROWB + 16 * ((2 * ks + g) ^ k_swz<D>(l32));
    }
    // K^T: rows 16*ks + 4*g + 8*h + rt (keys in the C-layout order of dS^T),
    // columns 32*mb + ct .. +3
    const int rt = (lane & 15) >> 2;
    const int ct = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    int kto[2][D / 32];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int mb = 0; mb < D / 32; ++mb) {
            const int row = 4 * g + 8 * h + rt, col = 32 * mb + ct;
            kto[h][mb] = row * ROWB + 16 * ((col >> 3) ^ rt_swz<D>(row)) + 2 * (col & 7);
        }
    const int last_visible = CAUSAL ? min(qrow, N - 1) : N - 1;

    f32x16 dqt[D / 32];
#pragma unroll
    for (int mb = 0; mb < D / 32; ++mb) dqt[mb] = zero16();

    auto step = [&](int kt, const char* Ks, const char* Vs, char* kn, char* vn) __attribute__((always_inline)) {
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (kt + 1 < nkt) issue(kt + 1, kn, vn);
        if (kt >= nkt_w) return;
        // S^T = K Q^T and dP^T = V dO^T (keys x queries)
        f32x16 st[NKB], pt[NKB];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            st[kb] = zero16();
            pt[kb] = zero16();
        }
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks)
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                st[kb] = mfma_bf16(*reinterpret_cast<const bf16x8*>(Ks + 32 * kb * ROWB + ko[ks]), qf[ks], st[kb]);
                pt[kb] = mfma_bf16(*reinterpret_cast<const bf16x8*>(Vs + 32 * kb * ROWB + vo[ks]), df[ks], pt[kb]);
            }
        // Mask, only on tiles that cross the diagonal or the end: masked
        // scores become -inf, so P = 2^(-inf) = 0 below.  Kept out of the dS
        // loop, which would otherwise carry a compare and a select per element
        // on every tile.
        const bool need_mask = (kt * BC + BC > N) || (CAUSAL && kt * BC + BC - 1 > wrow0);
        if (need_mask) {
            const int lim = last_visible - kt * BC - 4 * g;
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    if (32 * kb + 8 * (r >> 2) + (r & 3) > lim) st[kb][r] = -INFINITY;
        }
        // dS^T = P^T (dP^T - D), P^T = 2^(c S^T - LSE log2 e)
        bf16x8 sb[BC / 16];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                uint32_t pk[4];
#pragma unroll
                for (int j = 0; j < 8; j += 2) {
                    float v2[2];
#pragma unroll
                    for (int t = 0; t < 2; ++t) {
                        const int r = 8 * h + j + t;
                        const float p = exp2_fast(fmaf(st[kb][r], c, -lse2));
                        v2[t] = p * (pt[kb][r] - dd);
                    }
                    pk[j / 2] = pack_bf16x2(v2[0], v2[1]);
                }
                sb[2 * kb + h] = as_bf16x8(make_uint4(pk[0], pk[1], pk[2], pk[3]));
            }
        // dQ^T += K^T dS^T
#pragma unroll
        for (int ks = 0; ks < BC / 16; ++ks)
#pragma unroll
            for (int mb = 0; mb < D / 32; ++mb) {
                const uint2 lo = lds_read_tr16x4(Ks + 16 * ks * ROWB + kto[0][mb]);
                const uint2 hi = lds_read_tr16x4(Ks + 16 * ks * ROWB + kto[1][mb]);
                dqt[mb] = mfma_bf16(as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y)), sb[ks], dqt[mb]);
            }
        // K^T reads for the first DQ_AHEAD products go out before the dS
        // arithmetic; the rest of dS is interleaved with the products.
        {
            constexpr int n = (BC / 16) * (D / 32);
            __builtin_amdgcn_sched_group_barrier(0x100, 2 * DQ_AHEAD, 0);     // LDS reads
            __builtin_amdgcn_sched_group_barrier(0x002, DQ_VALU_FIRST, 0);    // VALU
#pragma unroll
            for (int i = 0; i < n - DQ_AHEAD; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);            // MFMA
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, DQ_VALU_EACH, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, DQ_AHEAD, 0);
        }
    };

    if (nkt > 0) issue(0, kb0, vb0);
    for (int kt = 0; kt < nkt; kt += 2) {
        step(kt, kb0, vb0, kb1, vb1);
        if (kt + 1 < nkt) step(kt + 1, kb1, vb1, kb0, vb0);
    }

    // dQ = scale * (dQ^T)^T: lane holds row qrow, dims in runs of 4.  (Staging
    // the rows through LDS for whole-row stores, as the dK/dV kernel does,
    // measured within noise here: two workgroups per CU hide the epilogue.)
    if (row_live) {
        __bf16* drow = dQ + hoff + (size_t)qrow * D;
#pragma unroll
        for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
            for (int rb = 0; rb < 4; ++rb) {
                const int d0 = 32 * mb + 8 * rb + 4 * g;
                *reinterpret_cast<uint2*>(drow + d0) =
                    make_uint2(pack_bf16x2(scale * dqt[mb][4 * rb], scale * dqt[mb][4 * rb + 1]),
                               pack_bf16x2(scale * dqt[mb][4 * rb + 2], scale * dqt[mb][4 * rb + 3]));
            }
    }
}

template <int D, bool CAUSAL>
hipError_t launch_kernels(const BwdArgs& a) {
    hipStream_t st = (hipStream_t)a.stream;
    const int BH = a.B * a.H;
    const int G = a.H / a.Hkv, BHkv = a.B * a.Hkv;
    // dQ first: it also writes D and the base-2 LSE that the dK/dV kernel reads
    const int nqt = (a.N + DQ_BR - 1) / DQ_BR;
    hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL>), dim3((unsigned)(nqt * BH)), dim3(256), 0, st,
                       (const __bf16*)a.q, (const __bf16*)a.k, (const __bf16*)a.v, (const __bf16*)a.dout, a.o,
                       a.o_bf16 ? 1 : 0, a.lse, a.delta, a.lse2, (__bf16*)a.dq, BH, G, a.N, nqt, a.scale * kLog2e,
                       a.scale);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int nkt = (a.N + BWD_BC - 1) / BWD_BC;
    if (a.split) {
        const int hpg = a.split, ngr = G / hpg;     // query heads per group, groups per K/V head
        if (hpg < 1 || G % hpg != 0) return hipErrorInvalidValue;
        hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL, true>), dim3((unsigned)(nkt * BHkv * ngr)), dim3(BWD_THREADS),
                           0, st, (const __bf16*)a.q, (const __bf16*)a.k, (const __bf16*)a.v, (const __bf16*)a.dout,
                           a.lse2, a.delta, (__bf16*)a.dk, (__bf16*)a.dv, a.pdk, a.pdv, BHkv, G, hpg, a.N,
                           a.scale * kLog2e, a.scale);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        const long long n8 = (long long)BHkv * a.N * (D / 8);
        hipLaunchKernelGGL((bwd_kv_reduce_kernel<D>), dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, st,
                           a.pdk, a.pdv, (__bf16*)a.dk, (__bf16*)a.dv, n8, ngr, a.N, a.scale);
    } else {
        hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL, false>), dim3((unsigned)(nkt * BHkv)), dim3(BWD_THREADS), 0,
                           st, (const __bf16*)a.q, (const __bf16*)a.k, (const __bf16*)a.v, (const __bf16*)a.dout,
                           a.lse2, a.delta, (__bf16*)a.dk, (__bf16*)a.dv, nullptr, nullptr, BHkv, G, G, a.N,
                           a.scale * kLog2e, a.scale);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd(const BwdArgs& a) {
    if (a.d == 64) return a.causal ? launch_kernels<64, true>(a) : launch_kernels<64, false>(a);
    if (a.d == 256) return a.causal ? launch_kernels<256, true>(a) : launch_kernels<256, false>(a);
    return a.causal ? launch_kernels<128, true>(a) : launch_kernels<128, false>(a);
}

}  // namespace fa
