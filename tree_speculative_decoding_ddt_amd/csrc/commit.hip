// Accepted-path commit: exact copies of the accepted rows' KV and of the deepest
// accepted row's recurrent/conv state into the committed buffers.
// Source: "DDTree on vLLM: candid research notes", sections "Why hybrid attention
// makes it hard" (only the accepted path is copied into the contiguous KV and
// recurrent buffers) and "Where the next step is" (explicit accepted-branch commit
// keyed by node ids); "From DDTree to drafter training", "The Architecture of
// DDTree" (the KV cache keeps only the accepted path).
//
// All copies move 16-byte words; every length is read on the device.  A sequence
// whose walk failed (acc_len < 0), whose accepted rows are not tree rows, or whose
// prefix would overflow Pmax is skipped by every copy kernel and finally reported
// with acc_len = -1; prefix_len is advanced by the last kernel only, after all copies
// have read it.
#include "common.h"
#include "launch.h"

namespace ddt {

constexpr int kLayersPerLaunch = 16;

struct KVTable {
  const uint8_t* k_tree[kLayersPerLaunch];
  const uint8_t* v_tree[kLayersPerLaunch];
  uint8_t* k_cache[kLayersPerLaunch];
  uint8_t* v_cache[kLayersPerLaunch];
};
struct GDNTable {
  const uint8_t* S_scratch[kLayersPerLaunch];
  uint8_t* S[kLayersPerLaunch];
  const uint8_t* conv_scratch[kLayersPerLaunch];
  uint8_t* conv_state[kLayersPerLaunch];
};

// Pmax is the capacity (max_blocks * page_size for a paged cache).  Every accepted row
// acc_rows[s][0..a] must be a tree row in [0, T); a paged cache also needs a valid page
// for every destination position P .. P+a.  A sequence that fails any check is not
// written by any copy kernel, and the last kernel reports it with acc_len = -1.
__device__ __forceinline__ bool commit_ok(const int32_t* acc_rows, const int32_t* acc_len,
                                          const int32_t* prefix_len, int s, int T, int Pmax, int Lp1,
                                          int& a, int& P, const PagedKV& pg = PagedKV{nullptr, 0, 0, 0}) {
  a = acc_len[s];
  P = prefix_len[s];
  if (!(a >= 0 && a < Lp1 && P >= 0 && P + a + 1 <= Pmax)) return false;
  for (int j = 0; j <= a; ++j) {
    const int r = acc_rows[(size_t)s * Lp1 + j];
    if (r < 0 || r >= T) return false;
  }
  if (pg.bt != nullptr)
    for (int b = P >> pg.lps; b <= (P + a) >> pg.lps; ++b) {
      const int id = pg.bt[(size_t)s * pg.maxb + b];
      if (id < 0 || id >= pg.npages) return false;
    }
  return true;
}

// grid (n, layers in this launch); row_vecs = D*esize/16 words per (head, row).
// Contiguous cache [n][Hkv][Pmax][D], or (pg.bt set) the page pool [pages][Hkv][ps][D].
__global__ void __launch_bounds__(256) commit_kv_kernel(KVTable tab, const int32_t* __restrict__ acc_rows,
                                                        const int32_t* __restrict__ acc_len,
                                                        const int32_t* __restrict__ prefix_len, int Hkv,
                                                        int T, int Pmax, int row_vecs, int Lp1, PagedKV pg) {
  const int s = blockIdx.x, layer = blockIdx.y;
  int a, P;
  if (!commit_ok(acc_rows, acc_len, prefix_len, s, T, Pmax, Lp1, a, P, pg)) return;
  const uint4* kt = reinterpret_cast<const uint4*>(tab.k_tree[layer]);
  const uint4* vt = reinterpret_cast<const uint4*>(tab.v_tree[layer]);
  uint4* kc = reinterpret_cast<uint4*>(tab.k_cache[layer]);
  uint4* vc = reinterpret_cast<uint4*>(tab.v_cache[layer]);
  const int total = (a + 1) * Hkv * row_vecs;
  for (int idx = threadIdx.x; idx < total; idx += blockDim.x) {
    const int w = idx % row_vecs;
    const int rest = idx / row_vecs;
    const int h = rest % Hkv;
    const int j = rest / Hkv;
    const int r = acc_rows[s * Lp1 + j];
    if (r < 0 || r >= T) continue;
    const size_t src = ((size_t)(s * Hkv + h) * T + r) * row_vecs + w;
    const size_t dst = (pg.bt != nullptr ? pg.row(s, h, Hkv, P + j) : (size_t)(s * Hkv + h) * Pmax + P + j) * row_vecs + w;
    kc[dst] = kt[src];
    vc[dst] = vt[src];
  }
}

// grid (n, layers, chunks); copies S (state_vecs words) then conv (conv_vecs words).
__global__ void __launch_bounds__(256) commit_gdn_kernel(GDNTable tab, const int32_t* __restrict__ acc_rows,
                                                         const int32_t* __restrict__ acc_len,
                                                         const int32_t* __restrict__ prefix_len, int T,
                                                         int Pmax, long state_vecs, long conv_vecs,
                                                         int Lp1, PagedKV pg) {
  const int s = blockIdx.x, layer = blockIdx.y;
  int a, P;
  if (!commit_ok(acc_rows, acc_len, prefix_len, s, T, Pmax, Lp1, a, P, pg)) return;
  const int r = acc_rows[s * Lp1 + a];
  if (r < 0 || r >= T) return;
  const uint4* Ss = reinterpret_cast<const uint4*>(tab.S_scratch[layer]) + ((size_t)s * T + r) * state_vecs;
  uint4* Sd = reinterpret_cast<uint4*>(tab.S[layer]) + (size_t)s * state_vecs;
  const uint4* Cs = reinterpret_cast<const uint4*>(tab.conv_scratch[layer]) + ((size_t)s * T + r) * conv_vecs;
  uint4* Cd = reinterpret_cast<uint4*>(tab.conv_state[layer]) + (size_t)s * conv_vecs;
  const long total = state_vecs + conv_vecs;
  const long per = (total + gridDim.z - 1) / gridDim.z;
  const long beg = per * blockIdx.z;
  const long end = beg + per < total ? beg + per : total;
  for (long i = beg + threadIdx.x; i < end; i += blockDim.x) {
    if (i < state_vecs) Sd[i] = Ss[i];
    else Cd[i - state_vecs] = Cs[i - state_vecs];
  }
}

__global__ void commit_finalize_kernel(const int32_t* __restrict__ acc_rows, int32_t* acc_len, int32_t* prefix_len,
                                       int n, int T, int Pmax, int Lp1, PagedKV pg) {
  const int s = blockIdx.x * blockDim.x + threadIdx.x;
  if (s >= n) return;
  int a, P;
  if (commit_ok(acc_rows, acc_len, prefix_len, s, T, Pmax, Lp1, a, P, pg)) prefix_len[s] = P + a + 1;
  else acc_len[s] = -1;
}

hipError_t launch_commit(const int32_t* acc_rows, int32_t* acc_len, int32_t* prefix_len,
                         const ddt_kv_layer* kv, int n_kv, int Hkv, int D, int Pmax, int kv_esize,
                         const ddt_gdn_layer* gdn, int n_gdn, int H, int dk, int dv, int C, int W,
                         int act_esize, int n, int T, int L, hipStream_t st, const PagedKV& pg) {
  const int Lp1 = L + 1;
  for (int l0 = 0; l0 < n_kv; l0 += kLayersPerLaunch) {
    const int cnt = n_kv - l0 < kLayersPerLaunch ? n_kv - l0 : kLayersPerLaunch;
    KVTable tab = {};
    for (int j = 0; j < cnt; ++j) {
      tab.k_tree[j] = static_cast<const uint8_t*>(kv[l0 + j].k_tree);
      tab.v_tree[j] = static_cast<const uint8_t*>(kv[l0 + j].v_tree);
      tab.k_cache[j] = static_cast<uint8_t*>(kv[l0 + j].k_cache);
      tab.v_cache[j] = static_cast<uint8_t*>(kv[l0 + j].v_cache);
    }
    hipLaunchKernelGGL(commit_kv_kernel, dim3(n, cnt), dim3(256), 0, st, tab, acc_rows, acc_len,
                       prefix_len, Hkv, T, Pmax, D * kv_esize / 16, Lp1, pg);
  }
  const long state_vecs = (long)H * dv * dk * 4 / 16;
  const long conv_vecs = (long)(W - 1) * C * act_esize / 16;
  const int chunks = (int)((state_vecs + conv_vecs + 4095) / 4096);
  for (int l0 = 0; l0 < n_gdn; l0 += kLayersPerLaunch) {
    const int cnt = n_gdn - l0 < kLayersPerLaunch ? n_gdn - l0 : kLayersPerLaunch;
    GDNTable tab = {};
    for (int j = 0; j < cnt; ++j) {
      tab.S_scratch[j] = reinterpret_cast<const uint8_t*>(gdn[l0 + j].S_scratch);
      tab.S[j] = reinterpret_cast<uint8_t*>(gdn[l0 + j].S);
      tab.conv_scratch[j] = static_cast<const uint8_t*>(gdn[l0 + j].conv_scratch);
      tab.conv_state[j] = static_cast<uint8_t*>(gdn[l0 + j].conv_state);
    }
    hipLaunchKernelGGL(commit_gdn_kernel, dim3(n, cnt, chunks), dim3(256), 0, st, tab, acc_rows,
                       acc_len, prefix_len, T, Pmax, state_vecs, conv_vecs, Lp1, pg);
  }
  hipLaunchKernelGGL(commit_finalize_kernel, dim3(cdiv(n, 64)), dim3(64), 0, st, acc_rows, acc_len, prefix_len, n, T, Pmax,
                     Lp1, pg);
  return hipGetLastError();
}

}  // namespace ddt
