// fa_api.cpp -- the C ABI declared in include/fa.h: argument validation,
// workspace sizing and dispatch to the kernel launchers.  Nothing is enqueued
// unless every check passes.
#include "fa.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "fa_internal.hpp"


namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool dims_ok(int B, int H, int N) { return B >= 1 && H >= 1 && N >= 1; }

bool head_dim_ok(int d) { return d == 64 || d == 128; }
// the bf16 forward, backward and decodes also run at d = 256 (fp32 forward and fp8 do not)
bool head_dim_ok_bf16(int d) { return head_dim_ok(d) || d == 256; }

bool scale_ok(float s) { return std::isfinite(s) && s > 0.f; }

// B*H*N*d must fit the 64-bit byte arithmetic used everywhere, and B*H*N the
// 32-bit row indices of the kernels.
bool total_ok(int B, int H, int N, int d) {
    const long long rows = (long long)B * H * N;
    return rows <= 0x7fffffffLL && rows * d <= (1LL << 50);
}

// Hkv K/V heads shared by H query heads in equal groups (Hkv = H: multi-head).
bool kv_ok(int H, int Hkv) { return Hkv >= 1 && Hkv <= H && H % Hkv == 0; }

// The bf16 kernels address one head's [N,d] tensor with 32-bit byte offsets.
bool head_fits_u32(int N, int d) { return (long long)N * d * 2 < (1LL << 32); }

fa_status_t from_hip(hipError_t e) { return e == hipSuccess ? FA_OK : FA_ERR_HIP; }

constexpr int kMaxSplits = 256;

int auto_splits(int B, int H, int Hkv, int L) {
    long long units, target, min_keys, max_s;
    if (fa::decode_group_path(B, H, Hkv)) {
        // grouped kernel: one wave per (b, cache head, chunk), four per
        // workgroup and one workgroup per CU (its tiles fill the LDS): aim
        // for ~1024 units, one round over the chip (measured better than two
        // rounds of shorter chunks).  Small batches split down to two 32-key
        // tiles per chunk, but into at most 64 chunks: measured at B1 Hkv8,
        // 64 chunks beat both 16 (L = 4K) and 128 (L = 16K).
        units = (long long)B * Hkv;
        target = 1024;
        min_keys = 64;
        max_s = 64;
    } else if (fa::decode_small_group(B, H, Hkv) != 0) {
        // small-group kernel: one workgroup per (b, cache head, chunk); about
        // 512 workgroups, chunks of at least 256 keys, at most 32 chunks
        // (measured at B1-B64, groups of 2-4, L = 8192: within 3% of the best
        // forced split count; for a paged cache too, at B4-B64 with 64- and
        // 256-token pages)
        units = (long long)B * Hkv;
        target = 512;
        min_keys = 256;
        max_s = 32;
    } else {
        // per-head kernel: at least ~4096 workgroups so every CU holds
        // several, with chunks of 512 keys or more (shorter chunks measured
        // slower at batch 1-4)
        units = (long long)B * H;
        target = 4096;
        min_keys = 512;
        max_s = kMaxSplits;
    }
    long long s = (target + units - 1) / units;
    const long long max_by_len = (L + min_keys - 1) / min_keys;
    if (s > max_by_len) s = max_by_len;
    if (s > max_s) s = max_s;
    if (s < 1) s = 1;
    return (int)s;
}

// Effective split count: chunks of ceil(L/S) keys rounded up to a multiple of
// 32 (a 32-key tile of the grouped kernel then never straddles a page of a
// paged cache), with no empty chunk for a cache of length L.
void split_plan(int L, int requested, int& splits, int& chunk) {
    chunk = (L + requested - 1) / requested;
    chunk = (chunk + 31) / 32 * 32;
    splits = (L + chunk - 1) / chunk;
}

bool pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }
int log2i(int x) {
    int r = 0;
    while ((1 << r) < x) ++r;
    return r;
}

}  // namespace

extern "C" {

const char* fa_status_string(fa_status_t s) {
    switch (s) {
        case FA_OK: return "FA_OK";
        case FA_ERR_NULL: return "FA_ERR_NULL: a required pointer is NULL";
        case FA_ERR_ARG:
            return "FA_ERR_ARG: a size is < 1 or too large, Hkv does not divide H, or scale is not finite and positive";
        case FA_ERR_UNSUPPORTED:
            return "FA_ERR_UNSUPPORTED: dtype / head-dim combination not built, or a bf16 head of 2^32 bytes or more";
        case FA_ERR_ALIGN: return "FA_ERR_ALIGN: a pointer is not 16-byte aligned";
        case FA_ERR_WORKSPACE: return "FA_ERR_WORKSPACE: workspace missing or too small";
        case FA_ERR_HIP: return "FA_ERR_HIP: the HIP runtime reported an error";
        case FA_ERR_SCRATCH_LIMIT:
            return "FA_ERR_SCRATCH_LIMIT: the call needs more scratch than the library's static buffer "
                   "(FA_NOALLOC_SCRATCH_BYTES) holds";
    }
    return "unknown fa_status_t";
}

fa_status_t fa_fwd(const void* q, const void* k, const void* v, void* o, fa_dtype_t o_dtype, float* lse,
                   int B, int H, int Hkv, int N, int d, fa_dtype_t in_dtype, int causal, float scale,
                   void* stream) {
    if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
    if (!dims_ok(B, H, N) || !kv_ok(H, Hkv) || !scale_ok(scale) || !total_ok(B, H, N, d)) return FA_ERR_ARG;
    if (in_dtype != FA_BF16 && in_dtype != FA_FP32) return FA_ERR_UNSUPPORTED;
    if (in_dtype == FA_BF16 ? !head_dim_ok_bf16(d) : !head_dim_ok(d)) return FA_ERR_UNSUPPORTED;
    if (o_dtype != FA_BF16 && o_dtype != FA_FP32) return FA_ERR_UNSUPPORTED;
    if (in_dtype == FA_FP32 && o_dtype != FA_FP32) return FA_ERR_UNSUPPORTED;
    if (in_dtype == FA_BF16 && !head_fits_u32(N, d)) return FA_ERR_UNSUPPORTED;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse)) return FA_ERR_ALIGN;
    fa::FwdArgs a{q, k, v, o, lse, B, H, Hkv, N, d, in_dtype == FA_BF16, o_dtype == FA_BF16, causal != 0, scale,
                  stream};
    return from_hip(fa::launch_fwd(a));
}

fa_status_t fa_fwd_fp8(const void* q, const void* k, const void* vt, float q_scale, float k_scale, float v_scale,
                       void* o, fa_dtype_t o_dtype, float* lse, int B, int H, int Hkv, int N, int d, int causal,
                       float scale, void* stream) {
    if (!q || !k || !vt || !o || !lse) return FA_ERR_NULL;
    if (!dims_ok(B, H, N) || !kv_ok(H, Hkv) || !scale_ok(scale) || !total_ok(B, H, N, d)) return FA_ERR_ARG;
    if (!scale_ok(q_scale) || !scale_ok(k_scale) || !scale_ok(v_scale)) return FA_ERR_ARG;
    if (!head_dim_ok(d) || !head_fits_u32(N, d)) return FA_ERR_UNSUPPORTED;
    if (o_dtype != FA_BF16 && o_dtype != FA_FP32) return FA_ERR_UNSUPPORTED;
    if (!aligned16(q) || !aligned16(k) || !aligned16(vt) || !aligned16(o) || !aligned16(lse)) return FA_ERR_ALIGN;
    fa::Fp8FwdArgs a{q, k, vt, q_scale, k_scale, v_scale, o, lse, B, H, Hkv, N, d, o_dtype == FA_BF16,
                     causal != 0, scale, stream};
    return from_hip(fa::launch_fwd_fp8(a));
}

// workspace layout: D [B,H,N] fp32 and LSE log2 e [B,H,N] fp32, each padded
// to 256 bytes; then, when the grouped-head split is taken (s query heads per
// workgroup), partial dK^T and dV^T rows [B*H/s, N, d] fp32 each
static size_t bwd_row_bytes(int B, int H, int N) {
    return ((size_t)B * H * N * sizeof(float) + 255) & ~(size_t)255;
}
static size_t bwd_delta_bytes(int B, int H, int N) { return 2 * bwd_row_bytes(B, H, N); }

size_t fa_bwd_workspace_bytes(int B, int H, int Hkv, int N, int d) {
    if (!dims_ok(B, H, N) || !kv_ok(H, Hkv) || d < 1 || !total_ok(B, H, N, d)) return 0;
    size_t n = bwd_delta_bytes(B, H, N);
    const int s = fa::bwd_split_heads(B, H, Hkv, N);     // query heads per split workgroup, 0: none
    if (s > 0) n += 2 * ((size_t)B * H / s) * N * d * sizeof(float);
    return n;
}

fa_status_t fa_bwd(const void* q, const void* k, const void* v, const void* o, fa_dtype_t o_dtype,
                   const float* lse, const void* dout, void* dq, void* dk, void* dv, void* workspace,
                   size_t workspace_bytes, int B, int H, int Hkv, int N, int d, fa_dtype_t in_dtype, int causal,
                   float scale, void* stream) {
    if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv) return FA_ERR_NULL;
    if (!dims_ok(B, H, N) || !kv_ok(H, Hkv) || !scale_ok(scale) || !total_ok(B, H, N, d)) return FA_ERR_ARG;
    if (!head_dim_ok_bf16(d) || in_dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
    if (o_dtype != FA_BF16 && o_dtype != FA_FP32) return FA_ERR_UNSUPPORTED;
    if (!head_fits_u32(N, d)) return FA_ERR_UNSUPPORTED;
    const void* ptrs[] = {q, k, v, o, lse, dout, dq, dk, dv};
    for (const void* p : ptrs)
        if (!aligned16(p)) return FA_ERR_ALIGN;
    const size_t need = fa_bwd_workspace_bytes(B, H, Hkv, N, d);
    if (!workspace || workspace_bytes < need) return FA_ERR_WORKSPACE;
    if (!aligned16(workspace)) return FA_ERR_ALIGN;
    float* delta = static_cast<float*>(workspace);
    float* lse2 = reinterpret_cast<float*>(static_cast<char*>(workspace) + bwd_row_bytes(B, H, N));
    const int split = fa::bwd_split_heads(B, H, Hkv, N);
    float* pdk = split ? reinterpret_cast<float*>(static_cast<char*>(workspace) + bwd_delta_bytes(B, H, N)) : nullptr;
    float* pdv = split ? pdk + ((size_t)B * H / split) * N * d : nullptr;
    fa::BwdArgs a{q, k, v, o, lse, dout, dq, dk, dv, delta, lse2, pdk, pdv, split, B, H, Hkv, N, d,
                  o_dtype == FA_BF16, causal != 0, scale, stream};
    return from_hip(fa::launch_bwd(a));
}

int fa_decode_num_splits(int B, int H, int Hkv, int L, int d) {
    (void)d;
    if (!dims_ok(B, H, L) || !kv_ok(H, Hkv)) return 1;
    int splits, chunk;
    split_plan(L, auto_splits(B, H, Hkv, L), splits, chunk);
    return splits;
}

size_t fa_decode_workspace_bytes(int B, int H, int Hkv, int L, int d, int num_splits) {
    if (!dims_ok(B, H, L) || !kv_ok(H, Hkv) || d < 1 || num_splits < 0 || !total_ok(B, H, L, d)) return 0;
    int splits, chunk;
    // num_splits = 0: the automatic plan, the same for fa_decode and
    // fa_decode_paged
    split_plan(L, num_splits == 0 ? auto_splits(B, H, Hkv, L) : (num_splits > L ? L : num_splits), splits,
               chunk);
    const size_t parts = (size_t)B * H * splits;
    const size_t o_bytes = parts * (size_t)d * sizeof(float);
    return ((o_bytes + 255) & ~(size_t)255) + parts * sizeof(float);
}

}  // extern "C"

namespace {

// Every check of fa_decode except the workspace's; nothing is enqueued.
fa_status_t decode_validate(const void* q, const void* k_cache, const void* v_cache, const void* o,
                            const float* lse, int B, int H, int Hkv, int L, int d, fa_dtype_t dtype,
                            int num_splits, float scale) {
    if (!q || !k_cache || !v_cache || !o) return FA_ERR_NULL;
    if (!dims_ok(B, H, L) || !kv_ok(H, Hkv) || !scale_ok(scale) || num_splits < 0 || num_splits > L ||
        !total_ok(B, H, L, d))
        return FA_ERR_ARG;
    if (!head_dim_ok_bf16(d) || dtype != FA_BF16 || !head_fits_u32(L, d)) return FA_ERR_UNSUPPORTED;
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(o)) return FA_ERR_ALIGN;
    if (lse && !aligned16(lse)) return FA_ERR_ALIGN;
    return FA_OK;
}

// Bytes of fp32 partials the contiguous-cache plan of this call needs (the
// same carving decode_launch does).
size_t decode_plan_bytes(int B, int H, int Hkv, int L, int d, int num_splits) {
    int splits, chunk;
    split_plan(L, num_splits == 0 ? auto_splits(B, H, Hkv, L) : num_splits, splits, chunk);
    const size_t parts = (size_t)B * H * splits;
    return ((parts * (size_t)d * sizeof(float) + 255) & ~(size_t)255) + parts * sizeof(float);
}

// Split plan, partial buffers carved from the workspace, launch.
fa_status_t decode_launch(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse,
                          void* workspace, int B, int H, int Hkv, int L, int d, int num_splits, float scale,
                          void* stream) {
    int splits, chunk;
    split_plan(L, num_splits == 0 ? auto_splits(B, H, Hkv, L) : num_splits, splits, chunk);
    const size_t parts = (size_t)B * H * splits;
    float* o_part = static_cast<float*>(workspace);
    float* lse_part = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                               (((parts * (size_t)d * sizeof(float)) + 255) & ~(size_t)255));
    fa::DecodeArgs a{q, k_cache, v_cache, o, lse, o_part, lse_part, B, H, Hkv, L, d, splits, chunk, scale, stream,
                     fa::Paging{}};   // contiguous cache: no block table
    return from_hip(fa::launch_decode(a));
}

}  // namespace

extern "C" {

fa_status_t fa_decode(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse,
                      void* workspace, size_t workspace_bytes, int B, int H, int Hkv, int L, int d,
                      fa_dtype_t dtype, int num_splits, float scale, void* stream) {
    const fa_status_t st = decode_validate(q, k_cache, v_cache, o, lse, B, H, Hkv, L, d, dtype, num_splits, scale);
    if (st != FA_OK) return st;
    const size_t need = fa_decode_workspace_bytes(B, H, Hkv, L, d, num_splits);
    if (!workspace || workspace_bytes < need) return FA_ERR_WORKSPACE;
    if (!aligned16(workspace)) return FA_ERR_ALIGN;
    return decode_launch(q, k_cache, v_cache, o, lse, workspace, B, H, Hkv, L, d, num_splits, scale, stream);
}

fa_status_t fa_decode_noalloc(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse,
                              int B, int H, int Hkv, int L, int d, fa_dtype_t dtype, int num_splits, float scale,
                              void* stream) {
    const fa_status_t st = decode_validate(q, k_cache, v_cache, o, lse, B, H, Hkv, L, d, dtype, num_splits, scale);
    if (st != FA_OK) return st;
    if (decode_plan_bytes(B, H, Hkv, L, d, num_splits) > (size_t)FA_NOALLOC_SCRATCH_BYTES)
        return FA_ERR_SCRATCH_LIMIT;
    void* scratch = nullptr;
    if (fa::decode_scratch(&scratch) != hipSuccess) return FA_ERR_HIP;
    return decode_launch(q, k_cache, v_cache, o, lse, scratch, B, H, Hkv, L, d, num_splits, scale, stream);
}

fa_status_t fa_decode_paged(const void* q, const void* k_pool, const void* v_pool, const int32_t* block_table,
                            const int32_t* seq_lens, void* o, float* lse, void* workspace, size_t workspace_bytes,
                            int B, int H, int Hkv, int num_pages, int page_size, int max_pages_per_seq, int d,
                            fa_dtype_t dtype, int num_splits, float scale, void* stream) {
    if (!q || !k_pool || !v_pool || !block_table || !seq_lens || !o) return FA_ERR_NULL;
    if (!dims_ok(B, H, 1) || !kv_ok(H, Hkv) || !scale_ok(scale) || num_pages < 1 || max_pages_per_seq < 1 ||
        num_splits < 0)
        return FA_ERR_ARG;
    const long long Lmax = (long long)max_pages_per_seq * page_size;
    if (!pow2(page_size) || page_size < 32 || page_size > (1 << 16) || Lmax > 0x7fffffffLL ||
        num_splits > Lmax || !total_ok(B, H, (int)Lmax, d) || (long long)B * max_pages_per_seq > 0x7fffffffLL)
        return FA_ERR_ARG;
    if (!head_dim_ok_bf16(d) || dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
    if (!aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool) || !aligned16(o)) return FA_ERR_ALIGN;
    if ((reinterpret_cast<uintptr_t>(block_table) & 3) || (reinterpret_cast<uintptr_t>(seq_lens) & 3))
        return FA_ERR_ALIGN;
    if (lse && !aligned16(lse)) return FA_ERR_ALIGN;
    const int L = (int)Lmax;
    const size_t need = fa_decode_workspace_bytes(B, H, Hkv, L, d, num_splits);
    if (!workspace || workspace_bytes < need) return FA_ERR_WORKSPACE;
    if (!aligned16(workspace)) return FA_ERR_ALIGN;
    int splits, chunk;
    split_plan(L, num_splits == 0 ? auto_splits(B, H, Hkv, L) : num_splits, splits, chunk);
    const size_t parts = (size_t)B * H * splits;
    float* o_part = static_cast<float*>(workspace);
    float* lse_part = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                               (((parts * (size_t)d * sizeof(float)) + 255) & ~(size_t)255));
    fa::DecodeArgs a{q, k_pool, v_pool, o, lse, o_part, lse_part, B, H, Hkv, L, d, splits, chunk, scale, stream,
                     fa::Paging{block_table, seq_lens, num_pages, max_pages_per_seq, log2i(page_size), Hkv}};
    return from_hip(fa::launch_decode(a));
}

}  // extern "C"
