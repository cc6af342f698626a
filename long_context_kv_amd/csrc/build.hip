// Tree construction kernels: RoPE table, level pooling (build) and decode
// append.  Node value = mean of the C children values (picx.dev Tree
// Construction, Eq. 1); node key = pooler of the C children keys (Pooler
// Distillation, Eq. 5).  Arithmetic is float32; nodes are rounded once to the
// storage dtype when stored, and every level reads the stored children.
#include <algorithm>

#include "recsa_common.hpp"
#include "recsa_kernels.hpp"
#include "recsa_pool.hpp"

namespace recsa {

// ------------------------------------------------------------ RoPE table
__global__ void __launch_bounds__(kBlock) rope_table_kernel(float* table, int d, int n_pos,
                                                            double theta) {
  const int half = d / 2;
  const int64_t n = static_cast<int64_t>(n_pos) * half;
  for (int64_t i = blockIdx.x * static_cast<int64_t>(kBlock) + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * kBlock) {
    const int phi = static_cast<int>(i / half);
    const int j = static_cast<int>(i % half);
    const double inv_freq = pow(theta, (-2.0 * j) / d);
    const double ang = static_cast<double>(phi) * inv_freq;
    table[2 * i] = static_cast<float>(cos(ang));
    table[2 * i + 1] = static_cast<float>(sin(ang));
  }
}

// Build nodes [n_lo, n_hi) of `level` for every (sequence, KV head): 16 nodes
// per workgroup of NT threads.  Few tiles (an incremental chunk) take 512
// threads, so each wave pools two nodes instead of four and the short grid
// finishes sooner; many tiles (a full build) take 256, which keeps more
// tiles resident per CU.  Results are identical either way.
constexpr int kBuildWideTiles = 1024;     // below this many tiles: 512 threads

template <int DT, int D, int NT>
__global__ void __launch_bounds__(NT) build_level_kernel(recsa_tree tr, recsa_pooler P,
                                                             int level, int64_t n_lo,
                                                             int64_t n_hi) {
  using T = typename Stor<DT>::T;
  constexpr int NODES = 16;
  __shared__ PoolSmem<DT, D, NODES> sm;
  const int j = blockIdx.y, b = blockIdx.z;
  const int64_t first = n_lo + static_cast<int64_t>(blockIdx.x) * NODES;
  const int n_valid = static_cast<int>(min<int64_t>(NODES, n_hi - first));
  const int64_t rows_up = level_rows_dev(tr.L_cap, level - 1);
  const int64_t rows = level_rows_dev(tr.L_cap, level);
  const int64_t head = static_cast<int64_t>(b) * tr.Hkv + j;
  const T* kc = static_cast<const T*>(tr.K[level - 1]) + (head * rows_up + first * kC) * D;
  const T* vc = static_cast<const T*>(tr.V[level - 1]) + (head * rows_up + first * kC) * D;
  T* ko = static_cast<T*>(tr.K[level]) + (head * rows + first) * D;
  T* vo = static_cast<T*>(tr.V[level]) + (head * rows + first) * D;
  T* kro = tr.Kr[level] ? static_cast<T*>(tr.Kr[level]) + (head * rows + first) * D : nullptr;
  // level 1 also writes its children's rotated rows Kr[0] (read here anyway)
  T* krc = (level == 1 && tr.Kr[0])
               ? static_cast<T*>(tr.Kr[0]) + (head * rows_up + first * kC) * D
               : nullptr;
  pool_tile<DT, D, NODES, NT>(kc, vc, ko, vo, kro, static_cast<int>(first % kC), tr.rope,
                              n_valid, P, sm, nullptr, krc);
}

// Rotated keys Kr[0] of the level-0 rows [tb, te): each thread rotates 8
// pairs (j, j + D/2) of one row with 16-byte loads and stores, so a row takes
// D/16 threads and a workgroup 256 * 16 / D rows.  The same float32 rotation
// as rotate_key_row, element for element.
template <int DT, int D>
__global__ void __launch_bounds__(kBlock) rotate_level0_kernel(recsa_tree tr, int64_t tb,
                                                               int64_t te) {
  using T = typename Stor<DT>::T;
  constexpr int H2 = D / 2;
  constexpr int TPR = H2 / 8;                        // threads per row
  constexpr int RPB = kBlock / TPR;                  // rows per workgroup
  const int64_t t = tb + static_cast<int64_t>(blockIdx.x) * RPB + threadIdx.x / TPR;
  if (t >= te) return;
  const int j0 = 8 * (threadIdx.x % TPR);
  const int64_t head = static_cast<int64_t>(blockIdx.z) * tr.Hkv + blockIdx.y;
  const int64_t off = (head * tr.L_cap + t) * D;
  const T* src = static_cast<const T*>(tr.K[0]) + off;
  T* dst = static_cast<T*>(tr.Kr[0]) + off;
  float x[8], y[8], cs[16];
  load_vec<DT, 8>(src + j0, x);
  load_vec<DT, 8>(src + H2 + j0, y);
  const float* rp = tr.rope + (static_cast<int64_t>(t % kC) * H2 + j0) * 2;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float4 v = *reinterpret_cast<const float4*>(rp + 4 * i);
    cs[4 * i] = v.x;
    cs[4 * i + 1] = v.y;
    cs[4 * i + 2] = v.z;
    cs[4 * i + 3] = v.w;
  }
  float xo[8], yo[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) rope_pair(x[e], y[e], cs[2 * e], cs[2 * e + 1], xo[e], yo[e]);
  store_vec8<DT>(dst + j0, xo);
  store_vec8<DT>(dst + H2 + j0, yo);
}

// Decode append: write row t, then complete each node whose last token is t.
template <int DT, int D>
__global__ void __launch_bounds__(kBlock) append_kernel(recsa_tree tr, recsa_pooler P,
                                                        const void* k_new, const void* v_new,
                                                        const int64_t* pos) {
  using T = typename Stor<DT>::T;
  __shared__ PoolSmem<DT, D, 1> sm;
  const int j = blockIdx.x, b = blockIdx.y;
  const int64_t head = static_cast<int64_t>(b) * tr.Hkv + j;
  const int64_t t = pos[b];
  {
    const T* ks = static_cast<const T*>(k_new) + head * D;
    const T* vs = static_cast<const T*>(v_new) + head * D;
    T* kd = static_cast<T*>(tr.K[0]) + (head * tr.L_cap + t) * D;
    T* vd = static_cast<T*>(tr.V[0]) + (head * tr.L_cap + t) * D;
    for (int i = threadIdx.x; i < D; i += kBlock) {
      kd[i] = ks[i];
      vd[i] = vs[i];
    }
    if (tr.Kr[0])
      rotate_key_row<DT, D>(ks, static_cast<T*>(tr.Kr[0]) + (head * tr.L_cap + t) * D,
                            static_cast<int>(t % kC), tr.rope, threadIdx.x, kBlock);
  }
  int64_t span = 1;
  for (int l = 1; l < tr.n_levels; ++l) {
    span *= kC;
    if ((t + 1) % span != 0) break;
    __threadfence();
    __syncthreads();
    const int64_t node = (t + 1) / span - 1;
    const int64_t rows_up = level_rows_dev(tr.L_cap, l - 1);
    const int64_t rows = level_rows_dev(tr.L_cap, l);
    const T* kc = static_cast<const T*>(tr.K[l - 1]) + (head * rows_up + node * kC) * D;
    const T* vc = static_cast<const T*>(tr.V[l - 1]) + (head * rows_up + node * kC) * D;
    T* ko = static_cast<T*>(tr.K[l]) + (head * rows + node) * D;
    T* vo = static_cast<T*>(tr.V[l]) + (head * rows + node) * D;
    T* kro = tr.Kr[l] ? static_cast<T*>(tr.Kr[l]) + (head * rows + node) * D : nullptr;
    pool_tile<DT, D, 1, kBlock>(kc, vc, ko, vo, kro, static_cast<int>(node % kC), tr.rope, 1, P,
                                sm);
    __syncthreads();
  }
}

// ------------------------------------------------------------- launchers
hipError_t launch_rope_table(float* table, int d, int n_pos, double theta, hipStream_t s) {
  const int64_t n = static_cast<int64_t>(n_pos) * (d / 2);
  const int grid = static_cast<int>(std::min<int64_t>((n + kBlock - 1) / kBlock, 4096));
  rope_table_kernel<<<grid, kBlock, 0, s>>>(table, d, n_pos, theta);
  return hipGetLastError();
}

template <int DT, int D>
static hipError_t build_impl(const recsa_tree& tr, const recsa_pooler& P, int64_t tb, int64_t te,
                             hipStream_t s) {
  if (tr.Kr[0]) {
    // the rotated-key copy of level 0, when kept: the level-1 pass writes the
    // rows of the nodes it completes ([16 n_lo, 16 n_hi) covers [tb, 16 n_hi));
    // this pass rotates the rest, the rows of a trailing incomplete node
    const int64_t covered =
        tr.n_levels > 1 ? std::min<int64_t>(te / kC, level_rows_host(tr.L_cap, 1)) * kC : tb;
    const int64_t rb = std::max<int64_t>(tb, covered);
    if (rb < te) {
      constexpr int RPB = kBlock / (D / 16);            // rows per workgroup
      dim3 grid(static_cast<unsigned>((te - rb + RPB - 1) / RPB), tr.Hkv, tr.B);
      rotate_level0_kernel<DT, D><<<grid, kBlock, 0, s>>>(tr, rb, te);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  int64_t span = 1;
  for (int l = 1; l < tr.n_levels; ++l) {
    span *= kC;
    const int64_t rows = level_rows_host(tr.L_cap, l);
    const int64_t n_lo = tb / span;
    const int64_t n_hi = std::min<int64_t>(te / span, rows);
    if (n_hi <= n_lo) continue;
    const int64_t tiles = (n_hi - n_lo + 15) / 16;
    dim3 grid(static_cast<unsigned>(tiles), tr.Hkv, tr.B);
    if (tiles * tr.Hkv * tr.B < kBuildWideTiles)
      build_level_kernel<DT, D, 512><<<grid, 512, 0, s>>>(tr, P, l, n_lo, n_hi);
    else
      build_level_kernel<DT, D, kBlock><<<grid, kBlock, 0, s>>>(tr, P, l, n_lo, n_hi);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_build(const recsa_tree& tr, const recsa_pooler& P, int64_t tb, int64_t te,
                        hipStream_t s) {
  if (tr.dtype == RECSA_BF16)
    return tr.d == 128 ? build_impl<RECSA_BF16, 128>(tr, P, tb, te, s)
                       : build_impl<RECSA_BF16, 64>(tr, P, tb, te, s);
  return tr.d == 128 ? build_impl<RECSA_F32, 128>(tr, P, tb, te, s)
                     : build_impl<RECSA_F32, 64>(tr, P, tb, te, s);
}

hipError_t launch_append(const recsa_tree& tr, const recsa_pooler& P, const void* k_new,
                         const void* v_new, const int64_t* pos, hipStream_t s) {
  dim3 grid(tr.Hkv, tr.B);
  if (tr.dtype == RECSA_BF16) {
    if (tr.d == 128)
      append_kernel<RECSA_BF16, 128><<<grid, kBlock, 0, s>>>(tr, P, k_new, v_new, pos);
    else
      append_kernel<RECSA_BF16, 64><<<grid, kBlock, 0, s>>>(tr, P, k_new, v_new, pos);
  } else {
    if (tr.d == 128)
      append_kernel<RECSA_F32, 128><<<grid, kBlock, 0, s>>>(tr, P, k_new, v_new, pos);
    else
      append_kernel<RECSA_F32, 64><<<grid, kBlock, 0, s>>>(tr, P, k_new, v_new, pos);
  }
  return hipGetLastError();
}

}  // namespace recsa
