// C ABI of libddt.so (declared in include/ddt.h): argument validation, workspace
// sizing and dispatch to the kernel launchers.  Validation happens entirely on the
// host and before any HIP call, so a rejected call touches no device state.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <mutex>

#include "common.h"
#include "launch.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = '\0';
  return DDT_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(DDT_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
int esize(int dt) { return dt == DDT_BF16 ? 2 : 4; }
bool dt_ok(int dt) { return dt == DDT_F32 || dt == DDT_BF16; }

#define DDT_NEED(ptr) \
  if ((ptr) == nullptr) return fail(DDT_ERR_ARG, "%s: null pointer '%s'", __func__, #ptr)
#define DDT_CHECK(cond, code, ...) \
  if (!(cond)) return fail(code, __VA_ARGS__)

}  // namespace

extern "C" {

const char* ddt_status_string(int status) {
  switch (status) {
    case DDT_OK: return "DDT_OK";
    case DDT_ERR_ARG: return "DDT_ERR_ARG";
    case DDT_ERR_UNSUPPORTED: return "DDT_ERR_UNSUPPORTED";
    case DDT_ERR_WORKSPACE: return "DDT_ERR_WORKSPACE";
    case DDT_ERR_HIP: return "DDT_ERR_HIP";
    default: return "DDT_ERR_UNKNOWN";
  }
}

const char* ddt_last_error(void) { return g_err; }

int ddt_abi_version(void) { return 1; }

// ---------------------------------------------------------------- tree build
static int build_args(int n, int L, int V, int B, int K, ddt::BuildPlan* plan) {
  DDT_CHECK(n >= 1 && L >= 1 && L <= 63 && V >= 1 && B >= 1 && B <= 64, DDT_ERR_ARG,
            "ddt_build_tree: need n>=1, 1<=L<=63, V>=1, 1<=B<=64 (got n=%d L=%d V=%d B=%d)", n, L, V, B);
  const int k = K == 0 ? B : K;
  DDT_CHECK(k >= 1 && k <= 64, DDT_ERR_ARG, "ddt_build_tree: K must be in [1, 64] (got %d)", K);
  DDT_CHECK(V <= (1 << 20), DDT_ERR_UNSUPPORTED, "ddt_build_tree: V=%d exceeds 2^20", V);
  const int keff = k < V ? k : V;
  *plan = ddt::plan_build_tree(n, L, V, B, keff);
  DDT_CHECK(plan->chunk <= 16384 && plan->cap / 2 >= keff, DDT_ERR_UNSUPPORTED,
            "ddt_build_tree: V=%d with K=%d does not fit the chunked top-K", V, k);
  return DDT_OK;
}

size_t ddt_build_tree_workspace(int n, int L, int V, int B, int K) {
  ddt::BuildPlan plan;
  if (build_args(n, L, V, B, K, &plan) != DDT_OK) return 0;
  return plan.total;
}

int ddt_build_tree(const void* draft_logits, int dt, int n, int L, int V, int B, int K, const int32_t* root_token,
                   int32_t* tok, int32_t* parent, int32_t* depth, float* score, uint64_t* anc, void* ws,
                   size_t ws_bytes, void* stream) {
  DDT_NEED(draft_logits); DDT_NEED(root_token); DDT_NEED(tok); DDT_NEED(parent);
  DDT_NEED(depth); DDT_NEED(score); DDT_NEED(anc); DDT_NEED(ws);
  DDT_CHECK(dt_ok(dt), DDT_ERR_UNSUPPORTED, "ddt_build_tree: dtype %d", dt);
  ddt::BuildPlan plan;
  const int st = build_args(n, L, V, B, K, &plan);
  if (st != DDT_OK) return st;
  DDT_CHECK(ws_bytes >= plan.total, DDT_ERR_WORKSPACE, "ddt_build_tree: workspace %zu < %zu bytes", ws_bytes,
            plan.total);
  DDT_CHECK(aligned16(ws), DDT_ERR_ARG, "ddt_build_tree: workspace not 16-byte aligned");
  return hip_status(ddt::launch_build_tree(draft_logits, dt, n, L, V, B, plan, root_token, tok, parent, depth,
                                           score, anc, ws, static_cast<hipStream_t>(stream)),
                    "ddt_build_tree");
}

// ---------------------------------------------------------------- tree build, no workspace argument
// For callers that cannot allocate (code under graph capture, tight serving loops): the
// tree build's scratch lives in a file-scope device array.  Its host-side name is not a
// device address; the address comes from hipGetSymbolAddress, once per device, with that
// device current, and only that pointer is handed to kernels.
namespace {
constexpr size_t kBuildScratchBytes = size_t(8) << 20;  // 8 MiB per device
constexpr int kMaxDevices = 64;
__device__ __align__(256) uint8_t scratch[kBuildScratchBytes];
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "ddt_build_tree_noalloc: hipGetDevice");
  DDT_CHECK(dev >= 0 && dev < kMaxDevices, DDT_ERR_ARG, "ddt_build_tree_noalloc: device %d above %d", dev,
            kMaxDevices - 1);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, "ddt_build_tree_noalloc: hipGetSymbolAddress");
    DDT_CHECK(p != nullptr, DDT_ERR_HIP, "ddt_build_tree_noalloc: no device address for the scratch array");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return DDT_OK;
}
}  // namespace

size_t ddt_build_tree_noalloc_max_scratch(void) { return kBuildScratchBytes; }

int ddt_build_tree_noalloc(const void* draft_logits, int dt, int n, int L, int V, int B, int K,
                           const int32_t* root_token, int32_t* tok, int32_t* parent, int32_t* depth, float* score,
                           uint64_t* anc, void* stream) {
  // the same host-side checks as ddt_build_tree, all before the first HIP call
  DDT_NEED(draft_logits); DDT_NEED(root_token); DDT_NEED(tok); DDT_NEED(parent);
  DDT_NEED(depth); DDT_NEED(score); DDT_NEED(anc);
  DDT_CHECK(dt_ok(dt), DDT_ERR_UNSUPPORTED, "ddt_build_tree_noalloc: dtype %d", dt);
  ddt::BuildPlan plan;
  const int st = build_args(n, L, V, B, K, &plan);
  if (st != DDT_OK) return st;
  DDT_CHECK(plan.total <= kBuildScratchBytes, DDT_ERR_WORKSPACE,
            "ddt_build_tree_noalloc: needs %zu bytes of scratch, above the static %zu (n=%d L=%d V=%d K=%d)",
            plan.total, kBuildScratchBytes, n, L, V, K);
  void* ws = nullptr;
  const int sa = scratch_address(&ws);
  if (sa != DDT_OK) return sa;
  return hip_status(ddt::launch_build_tree(draft_logits, dt, n, L, V, B, plan, root_token, tok, parent, depth,
                                           score, anc, ws, static_cast<hipStream_t>(stream)),
                    "ddt_build_tree_noalloc");
}

// ---------------------------------------------------------------- tree attention
static int attn_args(int n, int B, int Hq, int Hkv, int D, int Pmax, int dt) {
  DDT_CHECK(n >= 1 && B >= 0 && B <= 64 && Hq >= 1 && Hkv >= 1 && Pmax >= 0, DDT_ERR_ARG,
            "ddt_tree_attn: need n>=1, 0<=B<=64, Hq,Hkv>=1, Pmax>=0 (got n=%d B=%d Hq=%d Hkv=%d Pmax=%d)", n, B, Hq,
            Hkv, Pmax);
  DDT_CHECK(Hq % Hkv == 0 && Hq / Hkv <= 16, DDT_ERR_ARG, "ddt_tree_attn: Hq=%d must be a multiple of Hkv=%d, ratio <= 16",
            Hq, Hkv);
  DDT_CHECK(dt_ok(dt), DDT_ERR_UNSUPPORTED, "ddt_tree_attn: dtype %d", dt);
  DDT_CHECK(D == 64 || D == 128 || D == 256, DDT_ERR_UNSUPPORTED, "ddt_tree_attn: head size D=%d not built", D);
  return DDT_OK;
}

size_t ddt_tree_attn_workspace(int n, int B, int Hq, int Hkv, int D, int Pmax, int dt) {
  if (attn_args(n, B, Hq, Hkv, D, Pmax, dt) != DDT_OK) return 0;
  return ddt::plan_tree_attn(n, B, Hq, Hkv, D, Pmax, dt).total;
}

int ddt_tree_attn(const void* q, const void* k_cache, const void* v_cache, const int32_t* prefix_len,
                  const void* k_tree, const void* v_tree, const uint64_t* anc, int n, int B, int Hq, int Hkv, int D,
                  int Pmax, float scale, int dt, void* out, void* ws, size_t ws_bytes, void* stream) {
  DDT_NEED(q); DDT_NEED(k_cache); DDT_NEED(v_cache); DDT_NEED(prefix_len);
  DDT_NEED(k_tree); DDT_NEED(v_tree); DDT_NEED(anc); DDT_NEED(out);
  const int st = attn_args(n, B, Hq, Hkv, D, Pmax, dt);
  if (st != DDT_OK) return st;
  const ddt::AttnPlan plan = ddt::plan_tree_attn(n, B, Hq, Hkv, D, Pmax, dt);
  if (plan.total > 0) {
    DDT_NEED(ws);
    DDT_CHECK(ws_bytes >= plan.total, DDT_ERR_WORKSPACE, "ddt_tree_attn: workspace %zu < %zu bytes", ws_bytes,
              plan.total);
    DDT_CHECK(aligned16(ws), DDT_ERR_ARG, "ddt_tree_attn: workspace not 16-byte aligned");
  }
  DDT_CHECK(aligned16(q) && aligned16(k_cache) && aligned16(v_cache) && aligned16(k_tree) && aligned16(v_tree) &&
                aligned16(out),
            DDT_ERR_ARG, "ddt_tree_attn: tensors must be 16-byte aligned");
  const float sc = scale > 0.f ? scale : 1.f / sqrtf((float)D);
  return hip_status(ddt::launch_tree_attn(q, k_cache, v_cache, prefix_len, k_tree, v_tree, anc, n, B + 1, Hq, Hkv, D,
                                          Pmax, sc, dt, out, plan, ws, static_cast<hipStream_t>(stream)),
                    "ddt_tree_attn");
}

// ---------------------------------------------------------------- paged committed cache
static int paged_args(const char* fn, const int32_t* bt, int max_blocks, int page_size, int num_pages,
                      ddt::PagedKV& pg) {
  DDT_CHECK(bt != nullptr, DDT_ERR_ARG, "%s: block_table is NULL", fn);
  DDT_CHECK(page_size >= 1 && page_size <= 65536 && (page_size & (page_size - 1)) == 0, DDT_ERR_UNSUPPORTED,
            "%s: page_size=%d must be a power of two in [1, 65536]", fn, page_size);
  DDT_CHECK(max_blocks >= 1 && num_pages >= 1 && (long long)max_blocks * page_size <= (1ll << 30), DDT_ERR_ARG,
            "%s: need max_blocks, num_pages >= 1 and max_blocks*page_size <= 2^30 (got %d, %d, %d)", fn, max_blocks,
            num_pages, page_size);
  int lps = 0;
  while ((1 << lps) < page_size) ++lps;
  pg = ddt::PagedKV{bt, max_blocks, lps, num_pages};
  return DDT_OK;
}

size_t ddt_tree_attn_paged_workspace(int n, int B, int Hq, int Hkv, int D, int max_blocks, int page_size, int dt) {
  if (max_blocks < 1 || page_size < 1 || (long long)max_blocks * page_size > (1ll << 30)) return 0;
  return ddt_tree_attn_workspace(n, B, Hq, Hkv, D, max_blocks * page_size, dt);
}

int ddt_tree_attn_paged(const void* q, const void* k_pages, const void* v_pages, const int32_t* block_table,
                        int max_blocks, int page_size, int num_pages, const int32_t* prefix_len, const void* k_tree,
                        const void* v_tree, const uint64_t* anc, int n, int B, int Hq, int Hkv, int D, float scale,
                        int dt, void* out, void* ws, size_t ws_bytes, void* stream) {
  DDT_NEED(q); DDT_NEED(k_pages); DDT_NEED(v_pages); DDT_NEED(prefix_len);
  DDT_NEED(k_tree); DDT_NEED(v_tree); DDT_NEED(anc); DDT_NEED(out);
  ddt::PagedKV pg;
  int st = paged_args("ddt_tree_attn_paged", block_table, max_blocks, page_size, num_pages, pg);
  if (st != DDT_OK) return st;
  const int Pmax = max_blocks * page_size;
  st = attn_args(n, B, Hq, Hkv, D, Pmax, dt);
  if (st != DDT_OK) return st;
  const ddt::AttnPlan plan = ddt::plan_tree_attn(n, B, Hq, Hkv, D, Pmax, dt);
  if (plan.total > 0) {
    DDT_NEED(ws);
    DDT_CHECK(ws_bytes >= plan.total, DDT_ERR_WORKSPACE, "ddt_tree_attn_paged: workspace %zu < %zu bytes", ws_bytes,
              plan.total);
    DDT_CHECK(aligned16(ws), DDT_ERR_ARG, "ddt_tree_attn_paged: workspace not 16-byte aligned");
  }
  DDT_CHECK(aligned16(q) && aligned16(k_pages) && aligned16(v_pages) && aligned16(k_tree) && aligned16(v_tree) &&
                aligned16(out),
            DDT_ERR_ARG, "ddt_tree_attn_paged: tensors must be 16-byte aligned");
  const float sc = scale > 0.f ? scale : 1.f / sqrtf((float)D);
  return hip_status(ddt::launch_tree_attn(q, k_pages, v_pages, prefix_len, k_tree, v_tree, anc, n, B + 1, Hq, Hkv, D,
                                          Pmax, sc, dt, out, plan, ws, static_cast<hipStream_t>(stream), pg),
                    "ddt_tree_attn_paged");
}

// ---------------------------------------------------------------- tree attention with RoPE by depth
static size_t rope_q_bytes(int n, int B, int Hq, int D, int dt) {
  return ((size_t)n * (B + 1) * Hq * D * esize(dt) + 255) / 256 * 256;
}

size_t ddt_tree_attn_rope_workspace(int n, int B, int Hq, int Hkv, int D, int Pmax, int dt) {
  if (attn_args(n, B, Hq, Hkv, D, Pmax, dt) != DDT_OK) return 0;
  return rope_q_bytes(n, B, Hq, D, dt) + ddt::plan_tree_attn(n, B, Hq, Hkv, D, Pmax, dt).total;
}

int ddt_tree_rope(const void* q, const void* k_new, const void* v_new, const int32_t* depth, const int32_t* prefix_len,
                  int rot_dim, float theta, int n, int B, int Hq, int Hkv, int D, int dt, void* q_out, void* k_tree,
                  void* v_tree, void* stream) {
  DDT_NEED(q); DDT_NEED(k_new); DDT_NEED(v_new); DDT_NEED(depth); DDT_NEED(prefix_len);
  DDT_NEED(q_out); DDT_NEED(k_tree); DDT_NEED(v_tree);
  DDT_CHECK(n >= 1 && B >= 0 && B <= 64 && Hq >= 1 && Hkv >= 1, DDT_ERR_ARG,
            "ddt_tree_rope: need n>=1, 0<=B<=64, Hq,Hkv>=1");
  DDT_CHECK(dt_ok(dt), DDT_ERR_UNSUPPORTED, "ddt_tree_rope: dtype %d", dt);
  DDT_CHECK(D == 64 || D == 128 || D == 256, DDT_ERR_UNSUPPORTED, "ddt_tree_rope: head size D=%d not built", D);
  DDT_CHECK(rot_dim >= 16 && rot_dim <= D && rot_dim % 16 == 0, DDT_ERR_UNSUPPORTED,
            "ddt_tree_rope: rot_dim=%d must be a multiple of 16 in [16, D=%d]", rot_dim, D);
  DDT_CHECK(theta > 1.f && isfinite(theta), DDT_ERR_ARG, "ddt_tree_rope: theta=%g must be finite and > 1",
            (double)theta);
  DDT_CHECK(aligned16(q) && aligned16(k_new) && aligned16(v_new) && aligned16(q_out) && aligned16(k_tree) &&
                aligned16(v_tree),
            DDT_ERR_ARG, "ddt_tree_rope: tensors must be 16-byte aligned");
  return hip_status(ddt::launch_tree_rope(q, k_new, v_new, depth, prefix_len, n, B + 1, Hq, Hkv, D, rot_dim, theta,
                                          dt, q_out, k_tree, v_tree, static_cast<hipStream_t>(stream)),
                    "ddt_tree_rope");
}

int ddt_tree_attn_rope(const void* q, const void* k_new, const void* v_new, const int32_t* depth, int rot_dim,
                       float theta, const void* k_cache, const void* v_cache, const int32_t* prefix_len, void* k_tree,
                       void* v_tree, const uint64_t* anc, int n, int B, int Hq, int Hkv, int D, int Pmax, float scale,
                       int dt, void* out, void* ws, size_t ws_bytes, void* stream) {
  DDT_NEED(q); DDT_NEED(k_new); DDT_NEED(v_new); DDT_NEED(depth); DDT_NEED(k_cache); DDT_NEED(v_cache);
  DDT_NEED(prefix_len); DDT_NEED(k_tree); DDT_NEED(v_tree); DDT_NEED(anc); DDT_NEED(out); DDT_NEED(ws);
  const int st = attn_args(n, B, Hq, Hkv, D, Pmax, dt);
  if (st != DDT_OK) return st;
  DDT_CHECK(rot_dim >= 16 && rot_dim <= D && rot_dim % 16 == 0, DDT_ERR_UNSUPPORTED,
            "ddt_tree_attn_rope: rot_dim=%d must be a multiple of 16 in [16, D=%d]", rot_dim, D);
  DDT_CHECK(theta > 1.f && isfinite(theta), DDT_ERR_ARG, "ddt_tree_attn_rope: theta=%g must be finite and > 1",
            (double)theta);
  const size_t qb = rope_q_bytes(n, B, Hq, D, dt);
  const ddt::AttnPlan plan = ddt::plan_tree_attn(n, B, Hq, Hkv, D, Pmax, dt);
  DDT_CHECK(ws_bytes >= qb + plan.total, DDT_ERR_WORKSPACE, "ddt_tree_attn_rope: workspace %zu < %zu bytes", ws_bytes,
            qb + plan.total);
  DDT_CHECK(aligned16(ws) && aligned16(q) && aligned16(k_new) && aligned16(v_new) && aligned16(k_cache) &&
                aligned16(v_cache) && aligned16(k_tree) && aligned16(v_tree) && aligned16(out),
            DDT_ERR_ARG, "ddt_tree_attn_rope: tensors and workspace must be 16-byte aligned");
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  uint8_t* q_rot = static_cast<uint8_t*>(ws);
  hipError_t e = ddt::launch_tree_rope(q, k_new, v_new, depth, prefix_len, n, B + 1, Hq, Hkv, D, rot_dim, theta, dt,
                                       q_rot, k_tree, v_tree, hs);
  if (e != hipSuccess) return hip_status(e, "ddt_tree_attn_rope");
  const float sc = scale > 0.f ? scale : 1.f / sqrtf((float)D);
  return hip_status(ddt::launch_tree_attn(q_rot, k_cache, v_cache, prefix_len, k_tree, v_tree, anc, n, B + 1, Hq, Hkv,
                                          D, Pmax, sc, dt, out, plan, plan.total > 0 ? q_rot + qb : nullptr, hs),
                    "ddt_tree_attn_rope");
}

// ---------------------------------------------------------------- GDN tree step
static int gdn_args(int n, int B, int L, int H, int dk, int dv, int C, int W, int act_dt) {
  DDT_CHECK(n >= 1 && B >= 0 && B <= 64 && L >= 0 && H >= 1, DDT_ERR_ARG,
            "ddt_gdn_tree_step: need n>=1, 0<=B<=64, L>=0, H>=1 (got n=%d B=%d L=%d H=%d)", n, B, L, H);
  DDT_CHECK(L <= 63, DDT_ERR_ARG, "ddt_gdn_tree_step: depth bound L=%d exceeds 63", L);
  DDT_CHECK(dt_ok(act_dt), DDT_ERR_UNSUPPORTED, "ddt_gdn_tree_step: dtype %d", act_dt);
  DDT_CHECK(dk == dv && (dk == 32 || dk == 64 || dk == 128), DDT_ERR_UNSUPPORTED,
            "ddt_gdn_tree_step: dk=%d dv=%d not built (dk == dv in {32, 64, 128})", dk, dv);
  DDT_CHECK(W >= 2 && W <= 8, DDT_ERR_UNSUPPORTED, "ddt_gdn_tree_step: conv width W=%d not in [2, 8]", W);
  DDT_CHECK(C == 2 * H * dk, DDT_ERR_ARG, "ddt_gdn_tree_step: C=%d must equal 2*H*dk=%d", C, 2 * H * dk);
  return DDT_OK;
}

size_t ddt_gdn_tree_step_workspace(int n, int B, int H, int dk) {
  if (n < 1 || B < 0 || B > 64 || H < 1 || !(dk == 32 || dk == 64 || dk == 128)) return 0;
  return ddt::gdn_workspace(n, B + 1, H, dk);
}

int ddt_gdn_tree_step(const void* x, const float* conv_w, const void* conv_state, void* conv_scratch, const void* v,
                      const float* beta, const float* g, const float* S, float* S_scratch, void* o,
                      const int32_t* parent, int n, int B, int L, int H, int dk, int dv, int C, int W, int act_dt,
                      void* ws, size_t ws_bytes, void* stream) {
  DDT_NEED(x); DDT_NEED(conv_w); DDT_NEED(conv_state); DDT_NEED(v);
  DDT_NEED(beta); DDT_NEED(g); DDT_NEED(S); DDT_NEED(o); DDT_NEED(parent); DDT_NEED(ws);
  // S_scratch and conv_scratch may be NULL: nothing of the nodes' states is stored
  // (the commit then replays the accepted path, ddt_gdn_replay)
  const int st = gdn_args(n, B, L, H, dk, dv, C, W, act_dt);
  if (st != DDT_OK) return st;
  const size_t need = ddt::gdn_workspace(n, B + 1, H, dk);
  DDT_CHECK(ws_bytes >= need, DDT_ERR_WORKSPACE, "ddt_gdn_tree_step: workspace %zu < %zu bytes", ws_bytes, need);
  DDT_CHECK(aligned16(ws) && aligned16(S) && aligned16(S_scratch) && aligned16(x) && aligned16(conv_state) &&
                aligned16(conv_scratch),
            DDT_ERR_ARG, "ddt_gdn_tree_step: workspace, state and activation buffers must be 16-byte aligned");
  return hip_status(ddt::launch_gdn_tree_step(x, conv_w, conv_state, conv_scratch, v, beta, g, S, S_scratch, o,
                                              parent, n, B + 1, L, H, dk, C, W, act_dt, ws,
                                              static_cast<hipStream_t>(stream)),
                    "ddt_gdn_tree_step");
}

int ddt_gdn_tree_step_deferred(const void* x, const float* conv_w, const void* conv_state, void* conv_scratch,
                               const void* v, const float* beta, const float* g, const float* S, void* o,
                               const int32_t* parent, int n, int B, int L, int H, int dk, int dv, int C, int W,
                               int act_dt, void* ws, size_t ws_bytes, void* stream) {
  DDT_NEED(x); DDT_NEED(conv_w); DDT_NEED(conv_state); DDT_NEED(conv_scratch); DDT_NEED(v);
  DDT_NEED(beta); DDT_NEED(g); DDT_NEED(S); DDT_NEED(o); DDT_NEED(parent); DDT_NEED(ws);
  const int st = gdn_args(n, B, L, H, dk, dv, C, W, act_dt);
  if (st != DDT_OK) return st;
  DDT_CHECK(act_dt == DDT_BF16, DDT_ERR_UNSUPPORTED,
            "ddt_gdn_tree_step_deferred: built for bf16 activations (fp32 ones: ddt_gdn_tree_step)");
  const size_t need = ddt::gdn_workspace(n, B + 1, H, dk);
  DDT_CHECK(ws_bytes >= need, DDT_ERR_WORKSPACE, "ddt_gdn_tree_step_deferred: workspace %zu < %zu bytes", ws_bytes,
            need);
  DDT_CHECK(aligned16(ws) && aligned16(S) && aligned16(x) && aligned16(conv_state) && aligned16(conv_scratch),
            DDT_ERR_ARG, "ddt_gdn_tree_step_deferred: workspace, state and activation buffers must be 16-byte aligned");
  return hip_status(ddt::launch_gdn_tree_step_deferred(x, conv_w, conv_state, conv_scratch, v, beta, g, S, o, parent,
                                                       n, B + 1, H, dk, W, act_dt, ws,
                                                       static_cast<hipStream_t>(stream)),
                    "ddt_gdn_tree_step_deferred");
}

int ddt_gdn_tree_states(const float* S, float* S_scratch, int n, int B, int H, int dk, int dv, const void* ws,
                        size_t ws_bytes, void* stream) {
  DDT_NEED(S); DDT_NEED(S_scratch); DDT_NEED(ws);
  DDT_CHECK(n >= 1 && B >= 0 && B <= 64 && H >= 1, DDT_ERR_ARG,
            "ddt_gdn_tree_states: need n>=1, 0<=B<=64, H>=1 (got n=%d B=%d H=%d)", n, B, H);
  DDT_CHECK(dk == dv && (dk == 32 || dk == 64 || dk == 128), DDT_ERR_UNSUPPORTED,
            "ddt_gdn_tree_states: dk=%d dv=%d not built (dk == dv in {32, 64, 128})", dk, dv);
  const size_t need = ddt::gdn_workspace(n, B + 1, H, dk);
  DDT_CHECK(ws_bytes >= need, DDT_ERR_WORKSPACE, "ddt_gdn_tree_states: workspace %zu < %zu bytes", ws_bytes, need);
  DDT_CHECK(aligned16(ws) && aligned16(S) && aligned16(S_scratch), DDT_ERR_ARG,
            "ddt_gdn_tree_states: workspace and state buffers must be 16-byte aligned");
  return hip_status(ddt::launch_gdn_tree_states(S, S_scratch, n, B + 1, H, dk, ws, static_cast<hipStream_t>(stream)),
                    "ddt_gdn_tree_states");
}

// ---------------------------------------------------------------- GDN replay on commit
int ddt_gdn_replay(const int32_t* acc_rows, const int32_t* acc_len, const ddt_gdn_replay_layer* layers,
                   int n_layers, int H, int dk, int dv, int C, int W, int act_dt, int n, int B, int L,
                   void* stream) {
  DDT_NEED(acc_rows); DDT_NEED(acc_len);
  DDT_CHECK(n >= 1 && B >= 0 && B <= 64 && L >= 0 && L <= 63 && n_layers >= 0 && H >= 1, DDT_ERR_ARG,
            "ddt_gdn_replay: need n>=1, 0<=B<=64, 0<=L<=63, n_layers>=0, H>=1");
  DDT_CHECK(dt_ok(act_dt), DDT_ERR_UNSUPPORTED, "ddt_gdn_replay: dtype %d", act_dt);
  DDT_CHECK(dk == dv && (dk == 32 || dk == 64 || dk == 128), DDT_ERR_UNSUPPORTED,
            "ddt_gdn_replay: dk=%d dv=%d not built (dk == dv in {32, 64, 128})", dk, dv);
  DDT_CHECK(W >= 2 && W <= 8, DDT_ERR_UNSUPPORTED, "ddt_gdn_replay: conv width W=%d not in [2, 8]", W);
  DDT_CHECK(C == 2 * H * dk, DDT_ERR_ARG, "ddt_gdn_replay: C=%d must equal 2*H*dk=%d", C, 2 * H * dk);
  if (n_layers == 0) return DDT_OK;
  DDT_NEED(layers);
  for (int i = 0; i < n_layers; ++i) {
    const ddt_gdn_replay_layer& y = layers[i];
    DDT_CHECK(y.x && y.conv_w && y.v && y.beta && y.g && y.S && y.conv_state, DDT_ERR_ARG,
              "ddt_gdn_replay: null pointer in layer %d", i);
    DDT_CHECK(aligned16(y.S), DDT_ERR_ARG, "ddt_gdn_replay: S of layer %d not 16-byte aligned", i);
  }
  return hip_status(ddt::launch_gdn_replay(acc_rows, acc_len, layers, n_layers, H, dk, C, W, act_dt, n, B + 1, L,
                                           static_cast<hipStream_t>(stream)),
                    "ddt_gdn_replay");
}

// ---------------------------------------------------------------- tree walk
size_t ddt_tree_accept_workspace(int n, int B, int V) {
  if (n < 1 || B < 0 || B > 64 || V < 1) return 0;
  return ddt::plan_tree_accept(n, B, V).total;
}

int ddt_tree_accept(const void* target_logits, int dt, const int32_t* tok, const int32_t* parent, int n, int B, int L,
                    int V, int32_t* acc_rows, int32_t* acc_len, int32_t* bonus, void* ws, size_t ws_bytes,
                    void* stream) {
  DDT_NEED(target_logits); DDT_NEED(tok); DDT_NEED(parent); DDT_NEED(acc_rows);
  DDT_NEED(acc_len); DDT_NEED(bonus); DDT_NEED(ws);
  DDT_CHECK(n >= 1 && B >= 0 && B <= 64 && L >= 0 && L <= 63 && V >= 1, DDT_ERR_ARG,
            "ddt_tree_accept: need n>=1, 0<=B<=64, 0<=L<=63, V>=1 (got n=%d B=%d L=%d V=%d)", n, B, L, V);
  DDT_CHECK(dt_ok(dt), DDT_ERR_UNSUPPORTED, "ddt_tree_accept: dtype %d", dt);
  const ddt::AcceptPlan plan = ddt::plan_tree_accept(n, B, V);
  DDT_CHECK(ws_bytes >= plan.total, DDT_ERR_WORKSPACE, "ddt_tree_accept: workspace %zu < %zu bytes", ws_bytes,
            plan.total);
  DDT_CHECK(aligned16(ws), DDT_ERR_ARG, "ddt_tree_accept: workspace not 16-byte aligned");
  return hip_status(ddt::launch_tree_accept(target_logits, dt, tok, parent, n, B + 1, L, V, acc_rows, acc_len, bonus,
                                            plan, ws, static_cast<hipStream_t>(stream)),
                    "ddt_tree_accept");
}

int ddt_tree_accept_sampled(const void* target_logits, int dt, const float* gumbel, const float* temperature,
                            const int32_t* tok, const int32_t* parent, int n, int B, int L, int V, int32_t* acc_rows,
                            int32_t* acc_len, int32_t* bonus, void* ws, size_t ws_bytes, void* stream) {
  DDT_NEED(target_logits); DDT_NEED(gumbel); DDT_NEED(temperature); DDT_NEED(tok); DDT_NEED(parent);
  DDT_NEED(acc_rows); DDT_NEED(acc_len); DDT_NEED(bonus); DDT_NEED(ws);
  DDT_CHECK(n >= 1 && B >= 0 && B <= 64 && L >= 0 && L <= 63 && V >= 1, DDT_ERR_ARG,
            "ddt_tree_accept_sampled: need n>=1, 0<=B<=64, 0<=L<=63, V>=1 (got n=%d B=%d L=%d V=%d)", n, B, L, V);
  DDT_CHECK(dt_ok(dt), DDT_ERR_UNSUPPORTED, "ddt_tree_accept_sampled: dtype %d", dt);
  const ddt::AcceptPlan plan = ddt::plan_tree_accept(n, B, V);
  DDT_CHECK(ws_bytes >= plan.total, DDT_ERR_WORKSPACE, "ddt_tree_accept_sampled: workspace %zu < %zu bytes",
            ws_bytes, plan.total);
  DDT_CHECK(aligned16(ws), DDT_ERR_ARG, "ddt_tree_accept_sampled: workspace not 16-byte aligned");
  return hip_status(ddt::launch_tree_accept(target_logits, dt, tok, parent, n, B + 1, L, V, acc_rows, acc_len, bonus,
                                            plan, ws, static_cast<hipStream_t>(stream), gumbel, temperature),
                    "ddt_tree_accept_sampled");
}

// ---------------------------------------------------------------- commit
static int commit_impl(const int32_t* acc_rows, int32_t* acc_len, int32_t* prefix_len, const ddt_kv_layer* kv,
                       int n_kv, int Hkv, int D, int Pmax, int kv_dt, const ddt_gdn_layer* gdn, int n_gdn, int H,
                       int dk, int dv, int C, int W, int act_dt, int n, int B, int L, void* stream,
                       const ddt::PagedKV& pg) {
  DDT_NEED(acc_rows); DDT_NEED(acc_len); DDT_NEED(prefix_len);
  DDT_CHECK(n >= 1 && B >= 0 && B <= 64 && L >= 0 && L <= 63 && n_kv >= 0 && n_gdn >= 0, DDT_ERR_ARG,
            "ddt_commit: need n>=1, 0<=B<=64, 0<=L<=63, n_kv,n_gdn>=0");
  if (n_kv > 0) {
    DDT_NEED(kv);
    DDT_CHECK(dt_ok(kv_dt), DDT_ERR_UNSUPPORTED, "ddt_commit: kv dtype %d", kv_dt);
    DDT_CHECK(Hkv >= 1 && D >= 1 && Pmax >= 1 && (D * esize(kv_dt)) % 16 == 0, DDT_ERR_ARG,
              "ddt_commit: need Hkv,D,Pmax>=1 and D*elem %% 16 == 0 (Hkv=%d D=%d Pmax=%d)", Hkv, D, Pmax);
    for (int i = 0; i < n_kv; ++i) {
      DDT_CHECK(kv[i].k_tree && kv[i].v_tree && kv[i].k_cache && kv[i].v_cache, DDT_ERR_ARG,
                "ddt_commit: null pointer in kv layer %d", i);
      DDT_CHECK(aligned16(kv[i].k_tree) && aligned16(kv[i].v_tree) && aligned16(kv[i].k_cache) &&
                    aligned16(kv[i].v_cache),
                DDT_ERR_ARG, "ddt_commit: kv layer %d not 16-byte aligned", i);
    }
  }
  if (n_gdn > 0) {
    DDT_NEED(gdn);
    DDT_CHECK(dt_ok(act_dt), DDT_ERR_UNSUPPORTED, "ddt_commit: act dtype %d", act_dt);
    DDT_CHECK(H >= 1 && dk >= 1 && dv >= 1 && W >= 2 && C >= 1, DDT_ERR_ARG,
              "ddt_commit: need H,dk,dv,C>=1 and W>=2");
    DDT_CHECK(((long)H * dv * dk * 4) % 16 == 0 && ((long)(W - 1) * C * esize(act_dt)) % 16 == 0, DDT_ERR_ARG,
              "ddt_commit: state and conv rows must be whole 16-byte words");
    for (int i = 0; i < n_gdn; ++i) {
      DDT_CHECK(gdn[i].S_scratch && gdn[i].S && gdn[i].conv_scratch && gdn[i].conv_state, DDT_ERR_ARG,
                "ddt_commit: null pointer in gdn layer %d", i);
      DDT_CHECK(aligned16(gdn[i].S_scratch) && aligned16(gdn[i].S) && aligned16(gdn[i].conv_scratch) &&
                    aligned16(gdn[i].conv_state),
                DDT_ERR_ARG, "ddt_commit: gdn layer %d not 16-byte aligned", i);
    }
  }
  return hip_status(ddt::launch_commit(acc_rows, acc_len, prefix_len, kv, n_kv, Hkv, D, Pmax, esize(kv_dt), gdn,
                                       n_gdn, H, dk, dv, C, W, esize(act_dt), n, B + 1, L,
                                       static_cast<hipStream_t>(stream), pg),
                    "ddt_commit");
}

int ddt_commit(const int32_t* acc_rows, int32_t* acc_len, int32_t* prefix_len, const ddt_kv_layer* kv, int n_kv,
               int Hkv, int D, int Pmax, int kv_dt, const ddt_gdn_layer* gdn, int n_gdn, int H, int dk, int dv, int C,
               int W, int act_dt, int n, int B, int L, void* stream) {
  return commit_impl(acc_rows, acc_len, prefix_len, kv, n_kv, Hkv, D, Pmax, kv_dt, gdn, n_gdn, H, dk, dv, C, W,
                     act_dt, n, B, L, stream, ddt::PagedKV{nullptr, 0, 0, 0});
}

int ddt_commit_paged(const int32_t* acc_rows, int32_t* acc_len, int32_t* prefix_len, const ddt_kv_layer* kv,
                     int n_kv, int Hkv, int D, const int32_t* block_table, int max_blocks, int page_size,
                     int num_pages, int kv_dt, const ddt_gdn_layer* gdn, int n_gdn, int H, int dk, int dv, int C, int W,
                     int act_dt, int n, int B, int L, void* stream) {
  ddt::PagedKV pg;
  const int st = paged_args("ddt_commit_paged", block_table, max_blocks, page_size, num_pages, pg);
  if (st != DDT_OK) return st;
  return commit_impl(acc_rows, acc_len, prefix_len, kv, n_kv, Hkv, D, max_blocks * page_size, kv_dt, gdn, n_gdn, H,
                     dk, dv, C, W, act_dt, n, B, L, stream, pg);
}

}  // extern "C"
