// The C ABI used from C++ with plain device pointers (no Python, no torch):
// pool of an explicit size, page tables, the history written token by token
// with pkv_append_kv, then pkv_decode_attention_merged and, for comparison,
// pkv_decode_attention + pkv_merge_partials (which must give the same bits),
// and the per-step forms: the table written again from pinned host memory
// with pkv_page_table_write_async (no host wait, an event recorded after the
// copy) and decoded with pkv_decode_attention_merged_noalloc (no workspace):
// the same bits once more.  Then the live pool: the same histories in
// pinned host memory, an 8-page device pool, one step whose admission keeps
// each request's sink and newest pages resident and stages the rest, the
// last token appended again (same values) and written back: the same bits
// as the resident merged decode, and the host copy unchanged.
// Writes its inputs and results to the file named on the command line; the
// test that runs it compares them with the float64 oracle.
//
//   decode_from_c OUT_FILE
//
// File layout (little endian): int32 B, Hq, Hkv, D, ctx[B]; then q bf16
// [B][Hq][D]; K bf16 [B][Hkv][ctx_b][D] and V bf16 [B][Hkv][ctx_b][D] for
// each request in turn; then out fp32 [B][Hq][D] and lse fp32 [B][Hq].
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "../../include/pkv.h"

namespace {

int fail_pkv(const char* what, int rc) {
  std::fprintf(stderr, "%s failed: %d %s\n", what, rc, pkv_last_error());
  return 1;
}

#define HIP_OK(x)                                                              \
  do {                                                                         \
    hipError_t e_ = (x);                                                       \
    if (e_ != hipSuccess) {                                                    \
      std::fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(e_));            \
      return 1;                                                                \
    }                                                                          \
  } while (0)

uint64_t g_state = 0x9E3779B97F4A7C15ull;
// A bf16 value of about N(0, 1/3): the sum of three uniforms, rounded to
// nearest even.
uint16_t next_bf16() {
  float s = 0.f;
  for (int i = 0; i < 3; ++i) {
    g_state = g_state * 6364136223846793005ull + 1442695040888963407ull;
    s += (float)((g_state >> 40) & 0xFFFFFF) / 16777216.f - 0.5f;
  }
  uint32_t u;
  std::memcpy(&u, &s, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

}  // namespace

int main(int argc, char** argv) {
  if (argc != 2) {
    std::fprintf(stderr, "usage: %s OUT_FILE\n", argv[0]);
    return 2;
  }
  const int B = 3, Hq = 24, Hkv = 4, D = 256, PT = 64, TILE = 512, SLOTS = 4;
  const int ctx[B] = {700, 64, 1500};
  const int pt_stride = 32, num_pages = 40;
  const pkv_geom geom = {1, Hkv, D, PT};

  uint64_t page_bytes = 0;
  if (int rc = pkv_page_bytes(&geom, &page_bytes)) return fail_pkv("pkv_page_bytes", rc);
  void* arena = nullptr;
  HIP_OK(hipMalloc(&arena, page_bytes * num_pages));
  pkv_pool* pool = nullptr;
  if (int rc = pkv_pool_create(&geom, arena, page_bytes * num_pages, &pool))
    return fail_pkv("pkv_pool_create", rc);

  // page tables: the pages of a fixed shuffle, request by request
  std::vector<int32_t> perm(num_pages);
  for (int i = 0; i < num_pages; ++i) perm[i] = (i * 17 + 5) % num_pages;
  std::vector<int32_t> table(B * pt_stride, -1);
  int used = 0;
  for (int b = 0; b < B; ++b)
    for (int p = 0; p < (ctx[b] + PT - 1) / PT; ++p) table[b * pt_stride + p] = perm[used++];
  int32_t *d_table = nullptr, *d_ctx = nullptr, *d_pos = nullptr;
  HIP_OK(hipMalloc(&d_table, sizeof(int32_t) * B * pt_stride));
  HIP_OK(hipMalloc(&d_ctx, sizeof(int32_t) * B));
  HIP_OK(hipMalloc(&d_pos, sizeof(int32_t) * B));
  if (int rc = pkv_page_table_write(pool, table.data(), ctx, B, pt_stride, d_table, d_ctx, nullptr))
    return fail_pkv("pkv_page_table_write", rc);

  // the history, one token of every request per append call
  std::vector<std::vector<uint16_t>> K(B), V(B);
  for (int b = 0; b < B; ++b) {
    K[b].assign((size_t)Hkv * ctx[b] * D, 0);
    V[b].assign((size_t)Hkv * ctx[b] * D, 0);
  }
  uint16_t *d_k = nullptr, *d_v = nullptr;
  HIP_OK(hipMalloc(&d_k, sizeof(uint16_t) * B * Hkv * D));
  HIP_OK(hipMalloc(&d_v, sizeof(uint16_t) * B * Hkv * D));
  std::vector<uint16_t> kn(B * Hkv * D), vn(B * Hkv * D);
  std::vector<int32_t> pos(B);
  for (int t = 0; t < 1500; ++t) {
    for (int b = 0; b < B; ++b) {
      pos[b] = t < ctx[b] ? t : -1;
      for (int g = 0; g < Hkv; ++g)
        for (int d = 0; d < D; ++d) {
          const uint16_t k = next_bf16(), v = next_bf16();
          kn[(b * Hkv + g) * D + d] = k;
          vn[(b * Hkv + g) * D + d] = v;
          if (t < ctx[b]) {
            K[b][((size_t)g * ctx[b] + t) * D + d] = k;
            V[b][((size_t)g * ctx[b] + t) * D + d] = v;
          }
        }
    }
    HIP_OK(hipMemcpy(d_pos, pos.data(), sizeof(int32_t) * B, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(d_k, kn.data(), sizeof(uint16_t) * kn.size(), hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(d_v, vn.data(), sizeof(uint16_t) * vn.size(), hipMemcpyHostToDevice));
    if (int rc = pkv_append_kv(pool, 0, d_table, pt_stride, d_pos, B, d_k, d_v, nullptr))
      return fail_pkv("pkv_append_kv", rc);
  }

  std::vector<uint16_t> q((size_t)B * Hq * D);
  for (auto& x : q) x = next_bf16();
  uint16_t* d_q = nullptr;
  HIP_OK(hipMalloc(&d_q, sizeof(uint16_t) * q.size()));
  HIP_OK(hipMemcpy(d_q, q.data(), sizeof(uint16_t) * q.size(), hipMemcpyHostToDevice));

  // decode + merge in one call, then as two calls
  const size_t po_n = (size_t)B * Hq * SLOTS * D, pl_n = (size_t)B * Hq * SLOTS;
  float *d_po = nullptr, *d_pl = nullptr, *d_out = nullptr, *d_lse = nullptr;
  float *d_po2 = nullptr, *d_pl2 = nullptr, *d_out2 = nullptr, *d_lse2 = nullptr;
  HIP_OK(hipMalloc(&d_po, sizeof(float) * po_n));
  HIP_OK(hipMalloc(&d_pl, sizeof(float) * pl_n));
  HIP_OK(hipMalloc(&d_out, sizeof(float) * B * Hq * D));
  HIP_OK(hipMalloc(&d_lse, sizeof(float) * B * Hq));
  HIP_OK(hipMalloc(&d_po2, sizeof(float) * po_n));
  HIP_OK(hipMalloc(&d_pl2, sizeof(float) * pl_n));
  HIP_OK(hipMalloc(&d_out2, sizeof(float) * B * Hq * D));
  HIP_OK(hipMalloc(&d_lse2, sizeof(float) * B * Hq));
  pkv_decode_opts opts = {0, 256, 0};          // 256-token splits: the finalize runs too
  uint64_t ws_bytes = 0;
  if (int rc = pkv_decode_workspace_bytes(B, Hq, D, SLOTS * TILE, TILE, &opts, &ws_bytes))
    return fail_pkv("pkv_decode_workspace_bytes", rc);
  void* d_ws = nullptr;
  HIP_OK(hipMalloc(&d_ws, ws_bytes ? ws_bytes : 16));
  const float scale = 1.0f / 16.0f;
  if (int rc = pkv_decode_attention_merged(pool, 0, d_q, d_table, pt_stride, d_ctx, B, Hq,
                                           SLOTS * TILE, TILE, scale, d_po, d_pl, SLOTS, d_out,
                                           d_lse, d_ws, ws_bytes, &opts, nullptr))
    return fail_pkv("pkv_decode_attention_merged", rc);
  if (int rc = pkv_decode_attention(pool, 0, d_q, d_table, pt_stride, d_ctx, B, Hq, 0,
                                    SLOTS * TILE, TILE, scale, d_po2, d_pl2, SLOTS, d_ws,
                                    ws_bytes, &opts, nullptr))
    return fail_pkv("pkv_decode_attention", rc);
  if (int rc = pkv_merge_partials(d_po2, d_pl2, B * Hq, SLOTS, D, d_out2, d_lse2, nullptr))
    return fail_pkv("pkv_merge_partials", rc);
  HIP_OK(hipDeviceSynchronize());

  std::vector<float> out((size_t)B * Hq * D), lse((size_t)B * Hq), out2(out.size()),
      lse2(lse.size());
  HIP_OK(hipMemcpy(out.data(), d_out, sizeof(float) * out.size(), hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(lse.data(), d_lse, sizeof(float) * lse.size(), hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(out2.data(), d_out2, sizeof(float) * out2.size(), hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(lse2.data(), d_lse2, sizeof(float) * lse2.size(), hipMemcpyDeviceToHost));
  if (std::memcmp(out.data(), out2.data(), 4 * out.size()) ||
      std::memcmp(lse.data(), lse2.data(), 4 * lse.size())) {
    std::fprintf(stderr, "merged decode and decode + merge differ\n");
    return 1;
  }

  // the per-step forms: async table write from pinned memory, then the
  // no-allocation merged decode, queued with no host wait in between
  int32_t* h_table = nullptr;
  int32_t* h_ctx = nullptr;
  HIP_OK(hipHostMalloc(reinterpret_cast<void**>(&h_table), sizeof(int32_t) * B * pt_stride,
                       hipHostMallocDefault));
  HIP_OK(hipHostMalloc(reinterpret_cast<void**>(&h_ctx), sizeof(int32_t) * B,
                       hipHostMallocDefault));
  std::memcpy(h_table, table.data(), sizeof(int32_t) * B * pt_stride);
  std::memcpy(h_ctx, ctx, sizeof(int32_t) * B);
  HIP_OK(hipMemset(d_table, 0xFF, sizeof(int32_t) * B * pt_stride));   // forget the old table
  HIP_OK(hipMemset(d_ctx, 0, sizeof(int32_t) * B));
  hipEvent_t copied = nullptr;
  HIP_OK(hipEventCreateWithFlags(&copied, hipEventDisableTiming));
  if (int rc = pkv_page_table_write_async(pool, h_table, h_ctx, B, pt_stride, d_table, d_ctx,
                                          nullptr, copied))
    return fail_pkv("pkv_page_table_write_async", rc);
  if (int rc = pkv_decode_attention_merged_noalloc(pool, 0, d_q, d_table, pt_stride, d_ctx, B,
                                                   Hq, SLOTS * TILE, TILE, scale, d_po2, d_pl2,
                                                   SLOTS, d_out2, d_lse2, &opts, nullptr))
    return fail_pkv("pkv_decode_attention_merged_noalloc", rc);
  HIP_OK(hipEventSynchronize(copied));       // the pinned table may be reused from here
  HIP_OK(hipDeviceSynchronize());
  HIP_OK(hipMemcpy(out2.data(), d_out2, sizeof(float) * out2.size(), hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(lse2.data(), d_lse2, sizeof(float) * lse2.size(), hipMemcpyDeviceToHost));
  if (std::memcmp(out.data(), out2.data(), 4 * out.size()) ||
      std::memcmp(lse.data(), lse2.data(), 4 * lse.size())) {
    std::fprintf(stderr, "async table + no-allocation decode differ from the merged decode\n");
    return 1;
  }
  HIP_OK(hipEventDestroy(copied));
  HIP_OK(hipHostFree(h_table));
  HIP_OK(hipHostFree(h_ctx));

  // the live pool over a pinned host copy of the histories
  {
    const int LP = 8, SP = 32;
    void *larena = nullptr, *sarena = nullptr, *host = nullptr;
    HIP_OK(hipMalloc(&larena, page_bytes * LP));
    HIP_OK(hipMalloc(&sarena, page_bytes * SP));
    HIP_OK(hipHostMalloc(&host, page_bytes * num_pages, hipHostMallocMapped));
    HIP_OK(hipMemcpy(host, arena, page_bytes * num_pages, hipMemcpyDeviceToHost));
    pkv_pool *lpool = nullptr, *spool = nullptr;
    if (int rc = pkv_pool_create(&geom, larena, page_bytes * LP, &lpool))
      return fail_pkv("pkv_pool_create (live)", rc);
    if (int rc = pkv_pool_create(&geom, sarena, page_bytes * SP, &spool))
      return fail_pkv("pkv_pool_create (staging)", rc);
    int32_t* d_state = nullptr;
    HIP_OK(hipMalloc(&d_state, sizeof(int32_t) * B * (pt_stride + 2)));
    hipStream_t s_copy, s_compute, s_back;
    HIP_OK(hipStreamCreateWithFlags(&s_copy, hipStreamNonBlocking));
    HIP_OK(hipStreamCreateWithFlags(&s_compute, hipStreamNonBlocking));
    HIP_OK(hipStreamCreateWithFlags(&s_back, hipStreamNonBlocking));
    pkv_live* live = nullptr;
    if (int rc = pkv_live_create(lpool, spool, host, page_bytes * num_pages, B, pt_stride,
                                 d_state, s_copy, s_compute, s_back, &live))
      return fail_pkv("pkv_live_create", rc);
    const int32_t ids[B] = {10, 20, 30};
    const int32_t target[B] = {3, 2, 3};
    for (int b = 0; b < B; ++b)
      if (int rc = pkv_live_add(live, ids[b], target[b], 0)) return fail_pkv("pkv_live_add", rc);
    const int64_t lengths[B] = {ctx[0], ctx[1], ctx[2]};
    int32_t status[B];
    pkv_live_info info;
    if (int rc = pkv_live_step_begin(live, B, ids, lengths, table.data(), pt_stride, status,
                                     &info))
      return fail_pkv("pkv_live_step_begin", rc);
    for (int b = 0; b < B; ++b)
      if (status[b] == PKV_ADMIT_REFUSED_STEP) {
        std::fprintf(stderr, "request %d refused\n", b);
        return 1;
      }
    if (info.staged_pages <= 0 || info.resident_pages > LP) {
      std::fprintf(stderr, "unexpected step: %lld staged, %d resident\n",
                   (long long)info.staged_pages, info.resident_pages);
      return 1;
    }
    // the newest token of each request, appended again
    for (int b = 0; b < B; ++b)
      for (int g = 0; g < Hkv; ++g)
        for (int d = 0; d < D; ++d) {
          kn[(b * Hkv + g) * D + d] = K[b][((size_t)g * ctx[b] + ctx[b] - 1) * D + d];
          vn[(b * Hkv + g) * D + d] = V[b][((size_t)g * ctx[b] + ctx[b] - 1) * D + d];
        }
    HIP_OK(hipMemcpy(d_k, kn.data(), sizeof(uint16_t) * kn.size(), hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(d_v, vn.data(), sizeof(uint16_t) * vn.size(), hipMemcpyHostToDevice));
    if (int rc = pkv_live_layer(live, 0, d_q, d_k, d_v, Hq, TILE, scale, d_po2, d_pl2, SLOTS,
                                d_out2, d_lse2, d_ws, ws_bytes, &opts))
      return fail_pkv("pkv_live_layer", rc);
    HIP_OK(hipStreamSynchronize(s_compute));
    HIP_OK(hipStreamSynchronize(s_back));
    HIP_OK(hipMemcpy(out2.data(), d_out2, sizeof(float) * out2.size(), hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(lse2.data(), d_lse2, sizeof(float) * lse2.size(), hipMemcpyDeviceToHost));
    if (std::memcmp(out.data(), out2.data(), 4 * out.size()) ||
        std::memcmp(lse.data(), lse2.data(), 4 * lse.size())) {
      std::fprintf(stderr, "the live step differs from the resident merged decode\n");
      return 1;
    }
    std::vector<char> dev_copy(page_bytes * num_pages);
    HIP_OK(hipMemcpy(dev_copy.data(), arena, dev_copy.size(), hipMemcpyDeviceToHost));
    if (std::memcmp(dev_copy.data(), host, dev_copy.size())) {
      std::fprintf(stderr, "the host copy changed\n");
      return 1;
    }
    if (int rc = pkv_live_destroy(live)) return fail_pkv("pkv_live_destroy", rc);
    pkv_pool_destroy(lpool);
    pkv_pool_destroy(spool);
    HIP_OK(hipStreamDestroy(s_copy));
    HIP_OK(hipStreamDestroy(s_compute));
    HIP_OK(hipStreamDestroy(s_back));
    HIP_OK(hipFree(larena));
    HIP_OK(hipFree(sarena));
    HIP_OK(hipFree(d_state));
    HIP_OK(hipHostFree(host));
  }

  FILE* f = std::fopen(argv[1], "wb");
  if (!f) {
    std::fprintf(stderr, "cannot write %s\n", argv[1]);
    return 1;
  }
  const int32_t hdr[4] = {B, Hq, Hkv, D};
  std::fwrite(hdr, 4, 4, f);
  std::fwrite(ctx, 4, B, f);
  std::fwrite(q.data(), 2, q.size(), f);
  for (int b = 0; b < B; ++b) {
    std::fwrite(K[b].data(), 2, K[b].size(), f);
    std::fwrite(V[b].data(), 2, V[b].size(), f);
  }
  std::fwrite(out.data(), 4, out.size(), f);
  std::fwrite(lse.data(), 4, lse.size(), f);
  std::fclose(f);

  pkv_pool_destroy(pool);
  for (void* p : {(void*)arena, (void*)d_table, (void*)d_ctx, (void*)d_pos, (void*)d_k,
                  (void*)d_v, (void*)d_q, (void*)d_po, (void*)d_pl, (void*)d_out, (void*)d_lse,
                  (void*)d_po2, (void*)d_pl2, (void*)d_out2, (void*)d_lse2, d_ws})
    HIP_OK(hipFree(p));
  std::printf("ok\n");
  return 0;
}
