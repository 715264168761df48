// Internal launchers: one per kernel family, called by the C ABI in api.hip after
// validation.  Each returns the result of hipGetLastError() after its launches.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/ddt.h"

namespace ddt {

// ---- tree build
struct BuildPlan {
  int S;          // chunks per (sequence, depth) row
  int chunk;      // elements per chunk (multiple of 8)
  int K;          // candidates per depth
  int cap;        // candidate words a chunk may write: cap of 4 bytes (bf16), cap / 2 of 8 (fp32)
  size_t off_ckey, off_cid, off_stat, off_tid, off_tlp, total;
};
BuildPlan plan_build_tree(int n, int L, int V, int B, int K);
hipError_t launch_build_tree(const void* logits, int dt, int n, int L, int V, int B,
                             const BuildPlan& plan, const int32_t* root_token, int32_t* tok,
                             int32_t* parent, int32_t* depth, float* score, uint64_t* anc,
                             void* ws, hipStream_t st);

// ---- tree attention
struct AttnPlan {
  bool mfma;      // bf16 matrix-core path (else the scalar path, no workspace)
  int G, R, ntiles, nwg, nsplit, split_len;
  int units, grid;  // (sequence, kv head, split) units; blocks launched
  size_t off_lse, off_o, total;
};
AttnPlan plan_tree_attn(int n, int B, int Hq, int Hkv, int D, int Pmax, int dt);

// Paged committed cache: pool [num_pages][Hkv][2^lps][D]; position p of sequence s is
// slot p & (2^lps - 1) of page bt[s][p >> lps].  bt == nullptr: the contiguous cache.
// A page id outside [0, npages) is clamped into it (wrong data, never an access outside
// the pool); the commit refuses such a sequence instead.
struct PagedKV {
  const int32_t* bt;
  int maxb, lps, npages;
  __device__ __forceinline__ int page(int s, int p) const {
    const int pgid = bt[(size_t)s * maxb + (p >> lps)];
    return pgid < 0 ? 0 : (pgid >= npages ? npages - 1 : pgid);
  }
  // row index (in units of D elements) of position p of (s, kv head h) in the pool
  __device__ __forceinline__ size_t row(int s, int h, int Hkv, int p) const {
    return (((size_t)page(s, p) * Hkv + h) << lps) + (p & ((1 << lps) - 1));
  }
  // Rows of four wave-uniform positions: the four table entries come in through scalar
  // loads (lgkmcnt, so they do not join the vector-memory count of copies in flight),
  // all issued before one wait.  The addresses are first copied into scratch SGPRs by
  // scalar moves inside the asm, so each load reads SGPRs a scalar instruction wrote
  // (whatever wrote the operands before, e.g. a v_readlane spill reload).
  __device__ __forceinline__ void rows_uniform4(int s, int h, int Hkv, const int (&p)[4], size_t (&out)[4]) const {
    const int32_t* e[4];
    int pu[4], id[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pu[i] = __builtin_amdgcn_readfirstlane(p[i]);
      e[i] = bt + (size_t)s * maxb + (pu[i] >> lps);
    }
    uint64_t a0, a1, a2, a3;
    asm volatile(
        "s_mov_b64 %4, %8\n\ts_mov_b64 %5, %9\n\ts_mov_b64 %6, %10\n\ts_mov_b64 %7, %11\n\t"
        "s_load_dword %0, %4, 0x0\n\ts_load_dword %1, %5, 0x0\n\ts_load_dword %2, %6, 0x0\n\t"
        "s_load_dword %3, %7, 0x0\n\ts_waitcnt lgkmcnt(0)"
        : "=&s"(id[0]), "=&s"(id[1]), "=&s"(id[2]), "=&s"(id[3]), "=&s"(a0), "=&s"(a1), "=&s"(a2), "=&s"(a3)
        : "s"(e[0]), "s"(e[1]), "s"(e[2]), "s"(e[3]));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int g = id[i] < 0 ? 0 : (id[i] >= npages ? npages - 1 : id[i]);
      out[i] = (((size_t)g * Hkv + h) << lps) + (pu[i] & ((1 << lps) - 1));
    }
  }
};

hipError_t launch_tree_attn(const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* prefix_len, const void* k_tree, const void* v_tree,
                            const uint64_t* anc, int n, int T, int Hq, int Hkv, int D, int Pmax,
                            float scale, int dt, void* out, const AttnPlan& plan, void* ws,
                            hipStream_t st, const PagedKV& pg = PagedKV{nullptr, 0, 0, 0});

// ---- RoPE of the tree rows at prefix + depth (queries to q_out, keys/values to the tree scratch)
hipError_t launch_tree_rope(const void* q, const void* k_new, const void* v_new, const int32_t* depth,
                            const int32_t* prefix_len, int n, int T, int Hq, int Hkv, int D, int rot, float theta,
                            int dt, void* q_out, void* k_tree, void* v_tree, hipStream_t st);

// ---- GDN tree step
size_t gdn_workspace(int n, int T, int H, int dk);
hipError_t launch_gdn_tree_step(const void* x, const float* conv_w, const void* conv_state,
                                void* conv_scratch, const void* v, const float* beta,
                                const float* g, const float* S, float* S_scratch, void* o,
                                const int32_t* parent, int n, int T, int L, int H, int dk, int C,
                                int W, int act_dt, void* ws, hipStream_t st);

// ---- GDN tree step in chunk form (short conv included): without stored node states, or
// with them (then gdn_states_kernel writes them from what the chunk kernel leaves in
// kbuf / wbuf / gam / dep and the record tables of gdn_chunk_store_bytes())
hipError_t launch_gdn_chunk(const void* x, const float* conv_w, const void* conv_state, const void* v,
                            const float* beta, const float* g, const float* S, void* o, const int32_t* parent, int n,
                            int T, int H, int dk, int W, int act_dt, hipStream_t st);
size_t gdn_chunk_store_bytes(int n, int T, int H);
hipError_t launch_gdn_chunk_stored(const void* x, const float* conv_w, const void* conv_state, void* conv_scratch,
                                   const void* v, const float* beta, const float* g, const float* S, float* S_scratch,
                                   void* o, const int32_t* parent, int n, int T, int H, int dk, int W, int act_dt,
                                   float* kbuf, float* wbuf, float* gam, int32_t* dep, void* tables, hipStream_t st);
hipError_t launch_gdn_chunk_exports(const void* x, const float* conv_w, const void* conv_state, void* conv_scratch,
                                    const void* v, const float* beta, const float* g, const float* S, void* o,
                                    const int32_t* parent, int n, int T, int H, int dk, int W, int act_dt, float* kbuf,
                                    float* wbuf, float* gam, int32_t* dep, void* tables, hipStream_t st);
hipError_t launch_gdn_states(const float* S, float* S_scratch, int n, int T, int H, int dk, const float* kbuf,
                             const float* wbuf, const float* gam, const int32_t* dep, const void* tables,
                             hipStream_t st);
// the same split behind the C ABI (workspace of gdn_workspace(); see gdn_tree.hip)
hipError_t launch_gdn_tree_step_deferred(const void* x, const float* conv_w, const void* conv_state,
                                         void* conv_scratch, const void* v, const float* beta, const float* g,
                                         const float* S, void* o, const int32_t* parent, int n, int T, int H, int dk,
                                         int W, int act_dt, void* ws, hipStream_t st);
hipError_t launch_gdn_tree_states(const float* S, float* S_scratch, int n, int T, int H, int dk, const void* ws,
                                  hipStream_t st);

// ---- GDN replay on commit
hipError_t launch_gdn_replay(const int32_t* acc_rows, const int32_t* acc_len, const ddt_gdn_replay_layer* layers,
                             int n_layers, int H, int dk, int C, int W, int act_dt, int n, int T, int L,
                             hipStream_t st);

// ---- tree walk
struct AcceptPlan {
  int S;          // chunks per row for the argmax scan
  int chunk;
  size_t total;
};
AcceptPlan plan_tree_accept(int n, int B, int V);
hipError_t launch_tree_accept(const void* logits, int dt, const int32_t* tok,
                              const int32_t* parent, int n, int T, int L, int V,
                              int32_t* acc_rows, int32_t* acc_len, int32_t* bonus,
                              const AcceptPlan& plan, void* ws, hipStream_t st,
                              const float* gumbel = nullptr, const float* temperature = nullptr);

// ---- commit
hipError_t launch_commit(const int32_t* acc_rows, int32_t* acc_len, int32_t* prefix_len,
                         const ddt_kv_layer* kv, int n_kv, int Hkv, int D, int Pmax, int kv_esize,
                         const ddt_gdn_layer* gdn, int n_gdn, int H, int dk, int dv, int C, int W,
                         int act_esize, int n, int T, int L, hipStream_t st,
                         const PagedKV& pg = PagedKV{nullptr, 0, 0, 0});

}  // namespace ddt
