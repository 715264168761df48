// Branch-local short conv + Gated DeltaNet over the draft tree.
// Sources: "DDTree on vLLM: candid research notes", section "Why hybrid attention
// makes it hard": every node reads the recurrent (GDN) state and the short-conv
// state of its parent and writes its own to scratch, never to committed state;
// "The architecture of speculation", section "The DDTree Integration Challenge":
// recurrent state is per branch, not shared.
//
// Per node i (parent p; the committed state when p is not an earlier row), head h:
//   window = [conv state of p (W-1 rows), x_i];  y = SiLU(sum_j w[c][j] window[j][c])
//   q = y[q-channels of h] * dk^-1/2;  k = y[k-channels of h] / sqrt(|k|^2 + 1e-6)
//   S_i = g S_p + beta (v - g S_p k) k^T;  o_i = S_i q = g (S_p q) + beta (v - g S_p k) (k.q)
//
// Node states stored (S_scratch, conv_scratch), bf16 activations, T <= 65 and a depth
// bound L <= 16: the chunk form of gdn_chunk.hip (its kernel also writes the conv
// scratch and hands w, k and the path records over) and gdn_states_kernel, which writes
// every state from them.  Otherwise (fp32 activations, deeper bounds), two kernels:
//  gdn_conv   grid (n*T, heads/HG): a block per node and group of heads, dk/4 lanes per
//             head; gathers the node's conv window along its parent chain, writes the
//             conv scratch (exact copies), and leaves q (scaled), k (normalised) and k.q
//             in fp32 in the workspace.  Every node is independent here.
//  gdn_state  grid (n*H, dv/R): a block owns R rows of one head's [dv][dk] state, a
//             thread CPT columns of one row (groups of 4, so that a wave's 16-byte
//             stores cover whole row segments).  The block loads every node's
//             q, k, k.q, v, g, beta into LDS, reads the depth-first order the conv
//             kernel computed (largest subtree last), then walks the nodes with no
//             barrier: the parent's state is the node just visited or a branch point
//             held in a register stack of 8 slots (enough for any tree of up to 128
//             rows, whatever its depth).  Each node's state is written once to
//             S_scratch; nothing is re-read from memory.
#include <math.h>

#include "common.h"
#include "launch.h"

namespace ddt {

constexpr int kGdnMaxT = 128;
constexpr int kGdnMaxW = 8;

// Depth-first (pre-)order of one sequence's tree, computed in parallel over nodes by a
// block of >= Tn threads.  A row whose parent is not an earlier row starts a tree of its
// own (it reads the committed state).  Children are visited in increasing order of
// (subtree size, row), so the largest subtree comes last.  The walk keeps the state of
// a node with two or more children in a register stack slot while its earlier children
// are walked; a child that is not its parent's last one is "light" and its subtree holds
// fewer than half of its parent's nodes, so a node has at most log2(Tn) light edges
// above it and the slot index lvl (the count of those edges) stays below 8 for Tn <= 128
// whatever the depth.  Word k of the order describes the k-th node visited:
//   bits 0-7   node (row)
//   bits 8-9   source of the parent state: 0 committed, 1 the node just visited (a first
//              child), 2 stack slot `rslot` (a later child)
//   bits 12-14 rslot = lvl(parent)
//   bits 16-18 sslot = lvl(node), bit 20: save the node's state there (two or more children)
// While a later child of p is still to come, every node visited in between lies under a
// light child of p and has lvl > lvl(p), so slot lvl(p) still holds p's state when that
// child reads it.
__device__ void dfs_order(const int* par, int Tn, int* sz, int* nch, int* esib, int* lvl, int32_t* out) {
  const int tid = threadIdx.x;
  for (int u = tid; u < Tn; u += blockDim.x) sz[u] = nch[u] = 0;
  __syncthreads();
  int d_me = 0;
  if (tid < Tn) {
    int a = tid;
    while (true) {
      const int p = par[a];
      atomicAdd(&sz[a], 1);
      if (!(p >= 0 && p < a)) break;
      if (a == tid) atomicAdd(&nch[p], 1);
      a = p;
      ++d_me;
    }
  }
  __syncthreads();
  // esib: nodes of the siblings visited before this one; light: a sibling comes after it
  int light = 0;
  if (tid < Tn) {
    const int p = par[tid];
    const int vp = (p >= 0 && p < tid) ? p : -1;
    const int my = sz[tid];
    int e = 0;
    // branch-free and unrolled, so that the (broadcast) LDS reads of several j are in
    // flight together
#pragma unroll 8
    for (int j = 0; j < Tn; ++j) {
      const int pj = par[j], szj = sz[j];
      const int vpj = (pj >= 0 && pj < j) ? pj : -1;
      const bool sib = vpj == vp && j != tid;
      const bool before = szj < my || (szj == my && j < tid);
      e += sib && before ? szj : 0;
      light |= sib && !before;
    }
    esib[tid] = e;
    if (vp < 0) light = 0;  // the roots' order needs no stack: each reads the committed state
    lvl[tid] = light;       // this node's own edge; the chain sum follows
  }
  __syncthreads();
  int pos = 0, lv = 0;
  if (tid < Tn) {
    pos = d_me;
    int a = tid;
    while (true) {
      pos += esib[a];
      lv += lvl[a];
      const int p = par[a];
      if (!(p >= 0 && p < a)) break;
      a = p;
    }
  }
  __syncthreads();
  if (tid < Tn) lvl[tid] = lv;
  __syncthreads();
  if (tid < Tn) {
    const int p = par[tid];
    const bool rooted = !(p >= 0 && p < tid);
    const int src = rooted ? 0 : (esib[tid] == 0 ? 1 : 2);
    const int rslot = rooted ? 0 : lvl[p];
    out[pos] = tid | (src << 8) | (rslot << 12) | (lv << 16) | ((nch[tid] >= 2) << 20);
  }
}

// ------------------------------------------------------------------ conv + q/k
// N consecutive activations of one row as raw 32-bit words, moved in 16- or 8-byte chunks.
template <typename A, int N>
struct RowIO {
  static constexpr int WORDS = N * (int)sizeof(A) / 4;
  uint32_t w[WORDS];
  __device__ __forceinline__ void load(const A* p) {
    if constexpr (WORDS % 4 == 0) {
#pragma unroll
      for (int i = 0; i < WORDS / 4; ++i) {
        const uint4 c = reinterpret_cast<const uint4*>(p)[i];
        w[4 * i] = c.x; w[4 * i + 1] = c.y; w[4 * i + 2] = c.z; w[4 * i + 3] = c.w;
      }
    } else {
#pragma unroll
      for (int i = 0; i < WORDS / 2; ++i) {
        const uint2 c = reinterpret_cast<const uint2*>(p)[i];
        w[2 * i] = c.x; w[2 * i + 1] = c.y;
      }
    }
  }
  __device__ __forceinline__ void store(A* p) const {
    if constexpr (WORDS % 4 == 0) {
#pragma unroll
      for (int i = 0; i < WORDS / 4; ++i)
        reinterpret_cast<uint4*>(p)[i] = make_uint4(w[4 * i], w[4 * i + 1], w[4 * i + 2], w[4 * i + 3]);
    } else {
#pragma unroll
      for (int i = 0; i < WORDS / 2; ++i) reinterpret_cast<uint2*>(p)[i] = make_uint2(w[2 * i], w[2 * i + 1]);
    }
  }
  __device__ __forceinline__ float get(int e) const {
    if constexpr (sizeof(A) == 2) {
      const uint32_t x = w[e >> 1];
      return __uint_as_float((e & 1) ? (x & 0xffff0000u) : (x << 16));
    } else {
      return __uint_as_float(w[e]);
    }
  }
};

// Block = (sequence, node, group of HG heads); LPH lanes per head, each lane NC = 4 q
// channels and the same 4 k channels of its head.  The window's rows (newest first: the
// node, its parent, ... then committed conv-state rows) are resolved once per block.
// WT > 0 fixes the conv width at compile time: a lane's weights (4 channels x WT taps,
// contiguous) then come in 16-byte loads and the tap loop unrolls.
template <typename A, int DK, int WT>
__global__ void __launch_bounds__(256) gdn_conv_kernel(const A* __restrict__ x, const float* __restrict__ conv_w,
                                                       const A* __restrict__ conv_state, A* __restrict__ conv_scratch,
                                                       const int32_t* __restrict__ parent, int Tn, int H, int C,
                                                       int W_rt, float* __restrict__ qk, float* __restrict__ kq,
                                                       int32_t* __restrict__ order) {
  constexpr int NC = 4, LPH = DK / NC, HG = 256 / LPH;
  const int W = WT > 0 ? WT : W_rt;
  const int s = blockIdx.x / Tn, u = blockIdx.x % Tn;
  const int tid = threadIdx.x;
  __shared__ int par_s[kGdnMaxT];
  __shared__ int win[kGdnMaxW];  // back b: tree row (>= 0) or committed conv-state row j as -(1 + j)
  for (int i = tid; i < Tn; i += 256) par_s[i] = parent[(size_t)s * Tn + i];
  __syncthreads();
  if (tid == 0) {
    // back 0 is the node; then the parent chain; past the root come the committed
    // conv-state rows, newest (row W-2) first
    int cur = u, in_tree = 1, beyond = 0;
    for (int b = 0; b < W; ++b) {
      int r = u;
      if (b > 0) {
        if (in_tree) {
          const int p = par_s[cur];
          if (p >= 0 && p < cur) cur = p;
          else in_tree = 0;
        }
        r = in_tree ? cur : -(1 + (W - 1 - (++beyond)));
      }
      win[b] = r;
    }
  }
  __syncthreads();
  if (u == 0 && blockIdx.y == 0) {  // one block per sequence also orders its tree for the walk
    __shared__ int sz[kGdnMaxT], nch[kGdnMaxT], esib[kGdnMaxT], lvl[kGdnMaxT];
    dfs_order(par_s, Tn, sz, nch, esib, lvl, order + (size_t)s * Tn);
  }
  const int hp = blockIdx.y * HG + tid / LPH;
  if (hp >= H) return;
  const int j0 = (tid % LPH) * NC;
  const int cq = hp * DK + j0, ck = H * DK + hp * DK + j0;  // first q and k channel of this lane
  float yq[NC], yk[NC];
#pragma unroll
  for (int e = 0; e < NC; ++e) yq[e] = yk[e] = 0.f;
  auto tap_step = [&](int b, const float* wq, const float* wk) {  // wq/wk: this tap's weight per channel
    const int r = win[b];
    const A* src = r >= 0 ? x + ((size_t)s * Tn + r) * C : conv_state + ((size_t)s * (W - 1) + (-r - 1)) * C;
    RowIO<A, NC> vq, vk;
    vq.load(src + cq);
    vk.load(src + ck);
    if (b <= W - 2 && conv_scratch != nullptr) {
      A* dst = conv_scratch + (((size_t)s * Tn + u) * (W - 1) + (W - 2 - b)) * C;  // slot of back b
      vq.store(dst + cq);
      vk.store(dst + ck);
    }
#pragma unroll
    for (int e = 0; e < NC; ++e) {
      yq[e] += wq[e] * vq.get(e);
      yk[e] += wk[e] * vk.get(e);
    }
  };
  if constexpr (WT > 0) {
    float wq[NC][WT], wk[NC][WT];  // [channel][tap]: contiguous in conv_w
#pragma unroll
    for (int i = 0; i < NC * WT; i += 4) {
      const float4 a = *reinterpret_cast<const float4*>(conv_w + (size_t)cq * WT + i);
      const float4 c = *reinterpret_cast<const float4*>(conv_w + (size_t)ck * WT + i);
      const float av[4] = {a.x, a.y, a.z, a.w}, cv[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        wq[(i + t) / WT][(i + t) % WT] = av[t];
        wk[(i + t) / WT][(i + t) % WT] = cv[t];
      }
    }
#pragma unroll
    for (int b = 0; b < WT; ++b) {
      float tq[NC], tk[NC];
#pragma unroll
      for (int e = 0; e < NC; ++e) {
        tq[e] = wq[e][WT - 1 - b];
        tk[e] = wk[e][WT - 1 - b];
      }
      tap_step(b, tq, tk);
    }
  } else {
    for (int b = 0; b < W; ++b) {
      float tq[NC], tk[NC];
#pragma unroll
      for (int e = 0; e < NC; ++e) {
        tq[e] = conv_w[(size_t)(cq + e) * W + (W - 1 - b)];
        tk[e] = conv_w[(size_t)(ck + e) * W + (W - 1 - b)];
      }
      tap_step(b, tq, tk);
    }
  }
  float kk = 0.f, kqv = 0.f;
#pragma unroll
  for (int e = 0; e < NC; ++e) {
    yq[e] = yq[e] / (1.f + __expf(-yq[e]));
    yk[e] = yk[e] / (1.f + __expf(-yk[e]));
    kk += yk[e] * yk[e];
    kqv += yk[e] * yq[e];
  }
#pragma unroll
  for (int off = LPH / 2; off > 0; off >>= 1) {
    kk += __shfl_xor(kk, off, 64);
    kqv += __shfl_xor(kqv, off, 64);
  }
  const float rn = 1.f / sqrtf(kk + 1e-6f);
  const float qs = rsqrtf((float)DK);
  float* out = qk + (((size_t)s * Tn + u) * H + hp) * 2 * DK;
#pragma unroll
  for (int e = 0; e < NC; ++e) {
    out[j0 + e] = yq[e] * qs;
    out[DK + j0 + e] = yk[e] * rn;
  }
  if (tid % LPH == 0) kq[((size_t)s * Tn + u) * H + hp] = kqv * rn * qs;
}

// ------------------------------------------------------------------ state walk
typedef float fv4 __attribute__((ext_vector_type(4)));
typedef float fv8 __attribute__((ext_vector_type(8)));
template <int N> struct VecT;
template <> struct VecT<4> { typedef fv4 type; };
template <> struct VecT<8> { typedef fv8 type; };

// The stack of saved states (one CPT-wide vector per thread per slot) kept in registers:
// one named member per slot and a switch on the wave-uniform slot index, so no slot is
// ever addressed through memory.  8 slots cover every tree of up to 128 rows.
template <typename V> struct RegStack {
  V v0, v1, v2, v3, v4, v5, v6, v7;
  __device__ __forceinline__ V get(int i) const {
    switch (i) {
      case 0: return v0; case 1: return v1; case 2: return v2; case 3: return v3;
      case 4: return v4; case 5: return v5; case 6: return v6; default: return v7;
    }
  }
  __device__ __forceinline__ void put(int i, V x) {
    switch (i) {
      case 0: v0 = x; break; case 1: v1 = x; break; case 2: v2 = x; break; case 3: v3 = x; break;
      case 4: v4 = x; break; case 5: v5 = x; break; case 6: v6 = x; break; default: v7 = x; break;
    }
  }
};

// A thread's N columns of a row are N/4 groups of 4, the groups GS floats apart: with
// GS = DK/(N/4), each 16-byte store instruction of a wave covers whole row segments.
template <typename V, int N, int GS>
__device__ __forceinline__ V load_vec(const float* p) {
  V r;
#pragma unroll
  for (int j = 0; j < N / 4; ++j) {
    const float4 w = *reinterpret_cast<const float4*>(p + j * GS);
    r[4 * j] = w.x; r[4 * j + 1] = w.y; r[4 * j + 2] = w.z; r[4 * j + 3] = w.w;
  }
  return r;
}
// Streaming (non-temporal) stores: the per-node states are not read again in the round
// (the commit reads one of them), so they bypass the cache's write-allocate path.
template <typename V, int N, int GS>
__device__ __forceinline__ void store_vec_nt(float* p, V x) {
#pragma unroll
  for (int j = 0; j < N / 4; ++j) {
    const fv4 w = {x[4 * j], x[4 * j + 1], x[4 * j + 2], x[4 * j + 3]};
    __builtin_nontemporal_store(w, reinterpret_cast<fv4*>(p + j * GS));
  }
}

template <typename A, int DK, int CPT>
__global__ void __launch_bounds__(256) gdn_state_kernel(const float* __restrict__ qk, const float* __restrict__ kq,
                                                        const A* __restrict__ v, const float* __restrict__ beta,
                                                        const float* __restrict__ g, const float* __restrict__ S,
                                                        float* __restrict__ S_scratch, A* __restrict__ o,
                                                        const int32_t* __restrict__ order_g, int Tn, int H) {
  typedef typename VecT<CPT>::type V;
  constexpr int DV = DK;
  constexpr int LPR = DK / CPT;          // lanes per state row
  constexpr int R = 256 / LPR;           // state rows per block
  const int s = blockIdx.x / H, h = blockIdx.x % H;
  const int tid = threadIdx.x;
  const int rl = tid / LPR;
  const int r = blockIdx.y * R + rl;
  constexpr int GS = DK / (CPT / 4);      // stride between a thread's column groups
  const int c0 = (tid % LPR) * 4;          // first column of the thread's first group

  extern __shared__ float4 qk_s4[];      // [T][2*DK] floats: q then k of every node
  float* qk_s = reinterpret_cast<float*>(qk_s4);
  __shared__ float vv[kGdnMaxT][R];
  __shared__ float gb[kGdnMaxT][3];      // g, beta, k.q
  __shared__ int order[kGdnMaxT];

  // ---- inputs of every node into LDS (independent loads)
  const float4* qk4 = reinterpret_cast<const float4*>(qk);
  for (int idx = tid; idx < Tn * (2 * DK / 4); idx += 256) {
    const int u = idx / (2 * DK / 4), c = idx % (2 * DK / 4);
    qk_s4[idx] = qk4[(((size_t)s * Tn + u) * H + h) * (2 * DK / 4) + c];
  }
  for (int idx = tid; idx < Tn * R; idx += 256) {
    const int u = idx / R, j = idx % R;
    vv[u][j] = Elem<A>::load(v, (((size_t)s * Tn + u) * H + h) * DV + blockIdx.y * R + j);
  }
  for (int u = tid; u < Tn; u += 256) {
    const size_t ti = ((size_t)s * Tn + u) * H + h;
    gb[u][0] = g[ti];
    gb[u][1] = beta[ti];
    gb[u][2] = kq[ti];
    order[u] = order_g[(size_t)s * Tn + u];  // depth-first words from the conv kernel
  }
  // committed state slice of this thread (used by nodes at depth 0)
  const V sc = load_vec<V, CPT, GS>(&S[(((size_t)s * H + h) * DV + r) * DK + c0]);
  __syncthreads();

  // ---- walk (the next node's word is read while the current one is processed).  In
  // depth-first order a node's parent is either the node just processed (its state is
  // still in registers) or an earlier node with two or more children (kept in the stack
  // slot the order names); every row is processed, whatever its depth.
  RegStack<V> stk;
  V sprev = sc;
  int nxt = order[0];
  for (int k = 0; k < Tn; ++k) {
    const int cur = __builtin_amdgcn_readfirstlane(nxt);
    if (k + 1 < Tn) nxt = order[k + 1];
    const int u = cur & 0xff, src = (cur >> 8) & 3, rslot = (cur >> 12) & 7, sslot = (cur >> 16) & 7;
    const bool save = (cur >> 20) & 1;
    const V qv = load_vec<V, CPT, GS>(&qk_s[u * 2 * DK + c0]);
    const V kv = load_vec<V, CPT, GS>(&qk_s[u * 2 * DK + DK + c0]);
    const V sp = src == 0 ? sc : (src == 1 ? sprev : stk.get(rslot));
    float a = 0.f, b = 0.f;
#pragma unroll
    for (int e = 0; e < CPT; ++e) {
      a += sp[e] * kv[e];
      b += sp[e] * qv[e];
    }
    a = group_sum<LPR>(a);  // the row's LPR lanes: DPP lane moves, no LDS round trip
    b = group_sum<LPR>(b);
    const float gi = gb[u][0], bi = gb[u][1], kqi = gb[u][2], vi = vv[u][rl];
    const float delta = bi * (vi - gi * a);
    const V sn = gi * sp + delta * kv;
    if (save) stk.put(sslot, sn);
    sprev = sn;
    const size_t ti = ((size_t)s * Tn + u) * H + h;
    if (S_scratch != nullptr) store_vec_nt<V, CPT, GS>(&S_scratch[(ti * DV + r) * DK + c0], sn);
    if (c0 == 0) Elem<A>::store(o, ti * DV + r, gi * b + delta * kqi);
  }
}

// Workspace: q|k [n][T][H][2*dk] fp32, k.q [n][T][H], the depth-first order [n][T]; in the
// chunk form with stored states the same areas hold k and w, G_t and the depths, and the
// record tables follow.
size_t gdn_workspace(int n, int T, int H, int dk) {
  const size_t qk = (size_t)n * T * H * 2 * dk * sizeof(float);
  const size_t kq = (size_t)n * T * H * sizeof(float);
  const size_t ord = (size_t)n * T * sizeof(int32_t);
  return (qk + 255) / 256 * 256 + (kq + 255) / 256 * 256 + (ord + 255) / 256 * 256 + gdn_chunk_store_bytes(n, T, H);
}

// Where the chunk form with node states keeps its hand-over in the workspace (the areas of
// gdn_workspace()): k and w in the q|k area, G_t in the k.q area, the depths in the order
// area, then the record tables.
struct ChunkWs {
  float *k, *w, *gam;
  int32_t* dep;
  void* tables;
};
static ChunkWs chunk_ws(void* ws, int n, int T, int H, int dk) {
  const size_t qk_b = ((size_t)n * T * H * 2 * dk * sizeof(float) + 255) / 256 * 256;
  const size_t kq_b = ((size_t)n * T * H * sizeof(float) + 255) / 256 * 256;
  const size_t ord_b = ((size_t)n * T * sizeof(int32_t) + 255) / 256 * 256;
  uint8_t* b = static_cast<uint8_t*>(ws);
  ChunkWs c;
  c.k = reinterpret_cast<float*>(b);
  c.w = c.k + (size_t)n * T * H * dk;
  c.gam = reinterpret_cast<float*>(b + qk_b);
  c.dep = reinterpret_cast<int32_t*>(b + qk_b + kq_b);
  c.tables = b + qk_b + kq_b + ord_b;
  return c;
}

hipError_t launch_gdn_tree_step_deferred(const void* x, const float* conv_w, const void* conv_state,
                                         void* conv_scratch, const void* v, const float* beta, const float* g,
                                         const float* S, void* o, const int32_t* parent, int n, int T, int H, int dk,
                                         int W, int act_dt, void* ws, hipStream_t st) {
  const ChunkWs c = chunk_ws(ws, n, T, H, dk);
  return launch_gdn_chunk_exports(x, conv_w, conv_state, conv_scratch, v, beta, g, S, o, parent, n, T, H, dk, W,
                                  act_dt, c.k, c.w, c.gam, c.dep, c.tables, st);
}

hipError_t launch_gdn_tree_states(const float* S, float* S_scratch, int n, int T, int H, int dk, const void* ws,
                                  hipStream_t st) {
  const ChunkWs c = chunk_ws(const_cast<void*>(ws), n, T, H, dk);
  return launch_gdn_states(S, S_scratch, n, T, H, dk, c.k, c.w, c.gam, c.dep, c.tables, st);
}

// Depth bound up to which node states are formed from the chunk form.  The states
// kernel's work grows with each node's path length: on bushy trees (mean path about 5
// rows at L 15) it writes the states in 0.22 ms per call against the walk's 0.24, while
// trees whose nodes crowd the bound (a chain, a deep thin tree) cost it 0.25 ms at L 16
// and 0.29 at L 24.  Any tree is computed correctly either way: the bound only picks the
// path.
constexpr int kChunkStoreMaxL = 16;

template <typename A, int DK>
static hipError_t launch_gdn(const void* x, const float* conv_w, const void* conv_state, void* conv_scratch, const void* v,
                       const float* beta, const float* g, const float* S, float* S_scratch, void* o,
                       const int32_t* parent, int n, int T, int L, int H, int C, int W, void* ws, hipStream_t st) {
  constexpr int CPT = DK >= 64 ? 8 : 4;   // columns per thread
  constexpr int R = 256 / (DK / CPT);     // state rows per block
  const size_t qk_b = ((size_t)n * T * H * 2 * DK * sizeof(float) + 255) / 256 * 256;
  const size_t kq_b = ((size_t)n * T * H * sizeof(float) + 255) / 256 * 256;
  float* qk = static_cast<float*>(ws);
  float* kq = reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + qk_b);
  int32_t* ord = reinterpret_cast<int32_t*>(static_cast<uint8_t*>(ws) + qk_b + kq_b);
  if (S_scratch == nullptr && conv_scratch == nullptr && sizeof(A) == 2) {
    // no node state stored, bf16 activations: conv and delta rule in one kernel, in
    // chunk form on the matrix cores (the fp32 configuration keeps the walk, whose
    // rounding stays within its 1e-5 bound)
    return launch_gdn_chunk(x, conv_w, conv_state, v, beta, g, S, o, parent, n, T, H, DK, W, DDT_BF16, st);
  }
  if (S_scratch != nullptr && conv_scratch != nullptr && sizeof(A) == 2 && T <= 65 && W <= 8 &&
      L <= kChunkStoreMaxL) {
    // stored states, bf16 activations: the chunk form gives every node's w, then each
    // state is written by short-lived blocks (k and w in the q|k area, G_t in the k.q
    // area, depths in the order area)
    const ChunkWs c = chunk_ws(ws, n, T, H, DK);
    return launch_gdn_chunk_stored(x, conv_w, conv_state, conv_scratch, v, beta, g, S, S_scratch, o, parent, n, T, H,
                                   DK, W, DDT_BF16, c.k, c.w, c.gam, c.dep, c.tables, st);
  }
  const dim3 cgrid(n * T, (H + 256 / (DK / 4) - 1) / (256 / (DK / 4)));
  if (W == 4)
    hipLaunchKernelGGL((gdn_conv_kernel<A, DK, 4>), cgrid, dim3(256), 0, st, static_cast<const A*>(x), conv_w,
                       static_cast<const A*>(conv_state), static_cast<A*>(conv_scratch), parent, T, H, C, W, qk, kq, ord);
  else
    hipLaunchKernelGGL((gdn_conv_kernel<A, DK, 0>), cgrid, dim3(256), 0, st, static_cast<const A*>(x), conv_w,
                       static_cast<const A*>(conv_state), static_cast<A*>(conv_scratch), parent, T, H, C, W, qk, kq, ord);
  const size_t smem = (size_t)T * 2 * DK * sizeof(float);
  // the dynamic LDS limit is raised once per kernel, to the largest size any call uses
  // (a host-side attribute, not a stream operation: calls stay capturable in a graph)
  constexpr int kMaxSmem = 65 * 2 * DK * (int)sizeof(float);  // T <= 65 (B <= 64)
  auto kern = gdn_state_kernel<A, DK, CPT>;
  static const bool attr = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                               hipFuncAttributeMaxDynamicSharedMemorySize, kMaxSmem) == hipSuccess;
  (void)attr;
  hipLaunchKernelGGL(kern, dim3(n * H, DK / R), dim3(256), smem, st, qk, kq, static_cast<const A*>(v), beta, g, S,
                     S_scratch, static_cast<A*>(o), ord, T, H);
  return hipGetLastError();
}

hipError_t launch_gdn_tree_step(const void* x, const float* conv_w, const void* conv_state, void* conv_scratch,
                                const void* v, const float* beta, const float* g, const float* S, float* S_scratch,
                                void* o, const int32_t* parent, int n, int T, int L, int H, int dk, int C, int W,
                                int act_dt, void* ws, hipStream_t st) {
#define DDT_GDN(TY, DKV) \
  return launch_gdn<TY, DKV>(x, conv_w, conv_state, conv_scratch, v, beta, g, S, S_scratch, o, parent, n, T, L, H, C, W, ws, st)
  if (act_dt == DDT_BF16) {
    if (dk == 32) DDT_GDN(uint16_t, 32);
    if (dk == 64) DDT_GDN(uint16_t, 64);
    DDT_GDN(uint16_t, 128);
  }
  if (dk == 32) DDT_GDN(float, 32);
  if (dk == 64) DDT_GDN(float, 64);
  DDT_GDN(float, 128);
#undef DDT_GDN
}

}  // namespace ddt
