// fp32 prefill: block-sparse / BLASST flash attention on the vector ALUs.
//
// Full-precision path for float32 inputs (the fp32 static-window workload),
// with the same semantics as the bf16 MFMA path: the tile loops over its
// kept key blocks (DiT article section 3.3: the block list is consulted
// before any K/V load), keeps the online-softmax state per row (attention
// tutorial section 4.2; BLASST notes Algorithm 1) and, when lambda > 0,
// skips the exponent, the row-sum update, the V load and the P.V product of
// a block whose block max trails the running max by more than ln(lambda)
// in every row of the tile (BLASST notes section 3.1.1, section 4).
//
// One work-group per (batch, query head, query tile), one thread per query
// row.  K and V blocks of 64 keys are staged through LDS one after the other.

#include "device_common.h"
#include "internal.h"

namespace bsattn {
namespace {

constexpr int BC = 64;

template <int D, int BR>
__global__ __launch_bounds__(BR) void prefill_f32_kernel(const PrefillParams p) {
  __shared__ float tile[BC][D + 1];
  const int tid = threadIdx.x;
  int w = blockIdx.x;
  const int rank = w % p.Tr;
  w /= p.Tr;
  const int h = w % p.Hq;
  const int b = w / p.Hq;
  const int t = p.tile_order ? p.tile_order[rank] : (p.causal ? p.Tr - 1 - rank : rank);
  const int g = h / (p.Hq / p.Hkv);
  const int row = t * BR + tid;
  const bool row_ok = row < p.Nq;
  const float* qp = static_cast<const float*>(p.q);
  const float* kp = static_cast<const float*>(p.k) + (int64_t)b * p.ks_b + (int64_t)g * p.ks_h;
  const float* vp = static_cast<const float*>(p.v) + (int64_t)b * p.vs_b + (int64_t)g * p.vs_h;

  float q[D];
  for (int c = 0; c < D; ++c)
    q[c] = row_ok ? qp[(int64_t)b * p.qs_b + (int64_t)row * p.qs_t + (int64_t)h * p.qs_h + c] : 0.0f;
  float o[D];
  for (int c = 0; c < D; ++c) o[c] = 0.0f;
  float m_run = kNegInf, l = 0.0f;
  const bool dyn = p.lambda > 0.0f;
  const float ln_lambda = dyn ? logf(p.lambda) : kNegInf;

  // visited blocks: CSR list (or all), minus blocks wholly above the diagonal
  const int last_row = min(t * BR + BR, p.Nq) - 1;
  int beg = 0, end = p.Tc;
  if (p.row_ptr) {
    beg = p.row_ptr[t];
    end = p.row_ptr[t + 1];
  }
  if (p.causal) {  // ascending list: drop the entries wholly above the diagonal
    int n = beg;
    while (n < end && (p.row_ptr ? p.col_idx[n] : n) * BC <= last_row) ++n;
    end = n;
  }
  int visited = 0, skipped = 0, rows_agree = 0;
  for (int it = 0; it < end - beg; ++it) {
    const int e = p.block_order ? end - 1 - it : beg + it;  // descending: most recent keys first
    const int j = p.row_ptr ? p.col_idx[e] : e;
    ++visited;
    // stage K block
    __syncthreads();
    for (int x = tid; x < BC * D; x += BR) {
      const int r = x / D, c = x % D;
      const int key = j * BC + r;
      tile[r][c] = key < p.Nk ? kp[(int64_t)key * p.ks_t + c] : 0.0f;
    }
    __syncthreads();
    float s[BC];
    float m_blk = kNegInf;
    for (int r = 0; r < BC; ++r) {
      float acc = 0.0f;
      for (int c = 0; c < D; ++c) acc = fmaf(q[c], tile[r][c], acc);
      const int key = j * BC + r;
      const bool ok = row_ok && key < p.n_valid && (!p.causal || key <= row);
      s[r] = ok ? acc * p.scale : kNegInf;
      m_blk = fmaxf(m_blk, s[r]);
    }
    const float m_new = fmaxf(m_run, m_blk);
    bool skip = false;
    if (dyn) {
      const bool agree = (m_blk == kNegInf) || (m_blk - m_new < ln_lambda);
      skip = __syncthreads_and(agree) != 0;
      if (p.row_counters) rows_agree += __syncthreads_count(agree && row_ok);
    }
    if (p.block_state && tid == 0) {
      const int64_t bs = (((int64_t)b * p.Hq + h) * p.Tr + t) * p.Tc + j;
      p.block_state[bs] = skip ? 2 : 1;
    }
    if (skip) {
      ++skipped;
      m_run = m_new;
      continue;
    }
    const float alpha = (m_run == kNegInf) ? 0.0f : expf(m_run - m_new);
    const float m_use = (m_new == kNegInf) ? 0.0f : m_new;
    float rs = 0.0f;
    for (int r = 0; r < BC; ++r) {
      s[r] = expf(s[r] - m_use);  // exp(-inf) = 0 for disallowed keys
      rs += s[r];
    }
    l = alpha * l + rs;
    for (int c = 0; c < D; ++c) o[c] *= alpha;
    m_run = m_new;
    // stage V block (the K tile is no longer read)
    __syncthreads();
    for (int x = tid; x < BC * D; x += BR) {
      const int r = x / D, c = x % D;
      const int key = j * BC + r;
      tile[r][c] = key < p.Nk ? vp[(int64_t)key * p.vs_t + c] : 0.0f;
    }
    __syncthreads();
    for (int r = 0; r < BC; ++r) {
      const float pr = s[r];
      for (int c = 0; c < D; ++c) o[c] = fmaf(pr, tile[r][c], o[c]);
    }
  }
  if (row_ok) {
    float* op = static_cast<float*>(p.out) + (int64_t)b * p.os_b + (int64_t)row * p.os_t + (int64_t)h * p.os_h;
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
    for (int c = 0; c < D; ++c) op[c] = o[c] * inv;
    if (p.lse) p.lse[((int64_t)b * p.Hq + h) * p.Nq + row] = l > 0.0f ? m_run + logf(l) : kNegInf;
  }
  if (p.tile_counters && tid == 0) {
    int32_t* tc = p.tile_counters + 2 * ((((int64_t)b * p.Hq + h) * p.Tr) + t);
    tc[0] = visited;
    tc[1] = skipped;
  }
  if (p.row_counters && tid == 0) p.row_counters[((int64_t)b * p.Hq + h) * p.Tr + t] = rows_agree;
}

template <int D, int BR>
hipError_t launch(const PrefillParams& p, hipStream_t s) {
  const int64_t grid = (int64_t)p.B * p.Hq * p.Tr;
  hipLaunchKernelGGL((prefill_f32_kernel<D, BR>), dim3((unsigned)grid), dim3(BR), 0, s, p);
  return hipGetLastError();
}

}  // namespace

int launch_prefill_f32(const PrefillParams& p, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (p.d == 64) return p.Br == 64 ? launch<64, 64>(p, s) : launch<64, 128>(p, s);
  return p.Br == 64 ? launch<128, 64>(p, s) : launch<128, 128>(p, s);
}

}  // namespace bsattn
