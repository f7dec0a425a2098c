// Expert path for large batches (prefill): the gate/up and down projections
// of the activated experts as bf16 MFMA grouped GEMMs, plus an MFMA router.
//
// The layer ("Paper of the Week #3 - Half the FLOPs Is Not Half the Time",
// section "The Receipt", Eq. 2 for the weights; "Channel Selection for
// Mixture-of-Experts Decoding Needs No Calibration Data", section 2
// "Background" for the gated-MLP experts): for the tokens routed to expert e,
//   A_e = x[tokens of e]                       [n_e, H]  bf16
//   a   = silu(A_e Wg[e]^T) * (A_e Wu[e]^T) * w  [n_e, I] -> bf16
//   z   = a Wd[e]^T                             [n_e, H]  fp32 -> bf16
// and y[t] = sum of z over the token's k1 slots, in slot order, in fp32.
//
// Every product is "NT": both operands are stored K-contiguous (x and a rows
// along H / I, weight rows along H / I), which is the layout the MFMA
// operands want.  One tile engine serves all three GEMMs:
//   block = 256 threads = 4 waves in a 2x2 grid, tile BM x BN = 128 x 128,
//   K step 32 bf16; each wave owns a 64 x 64 sub-tile = 2 x 2 MFMA 32x32x16
//   (v_mfma_f32_32x32x16_bf16) accumulators; A and B K-slices are staged in
//   LDS (double buffered, rows padded by 16 bytes), the next slice's global
//   loads are in flight while the current one is multiplied.
// Lane layouts of v_mfma_f32_32x32x16_bf16 (checked on the device): lane l
// holds A row l%32 and B column l%32, k = 8*(l/32) .. +7; accumulator r of
// lane l is row (r/4)*8 + (l/32)*4 + r%4, column l%32.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {
namespace pf {

constexpr int kThreads = 256;
constexpr int BM = 128, BN = 128, BK = 32;
constexpr int LDS_ROW = BK + 8;  // bf16 elements per LDS row (16-byte pad)

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

struct Tile {
  uint16_t a[2][BM][LDS_ROW];
  uint16_t b[2][BN][LDS_ROW];
};

// Per thread: 2 of the 512 A chunks (16 B) and 2 of the 512 B chunks of one
// K slice.  Chunk c: row c / 4, k offset (c % 4) * 8.
struct Loader {
  const uint16_t *arow[2];
  const uint16_t *brow[2];
  int r[2], q[2];
  uint4 ra[2], rb[2];

  __device__ void fetch(int k0) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      ra[i] = ld16(arow[i] + k0 + q[i] * 8);
      rb[i] = ld16_stream(brow[i] + k0 + q[i] * 8);
    }
  }
  __device__ void store(Tile &T, int buf) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      *reinterpret_cast<uint4 *>(&T.a[buf][r[i]][q[i] * 8]) = ra[i];
      *reinterpret_cast<uint4 *>(&T.b[buf][r[i]][q[i] * 8]) = rb[i];
    }
  }
};

// acc[i][j] += A(wave rows i) * B(wave cols j)^T over one K slice in LDS.
__device__ __forceinline__ void mma_slice(const Tile &T, int buf, int wm, int wn,
                                          f32x16_t (&acc)[2][2]) {
  const int l = lane_id();
  const int lr = l & 31, lk = (l >> 5) * 8;
#pragma unroll
  for (int ks = 0; ks < BK; ks += 16) {
    bf16x8_t af[2], bf[2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
      af[i] = *reinterpret_cast<const bf16x8_t *>(&T.a[buf][wm * 64 + i * 32 + lr][ks + lk]);
#pragma unroll
    for (int j = 0; j < 2; ++j)
      bf[j] = *reinterpret_cast<const bf16x8_t *>(&T.b[buf][wn * 64 + j * 32 + lr][ks + lk]);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bf[j], acc[i][j], 0, 0, 0);
  }
}

// Full K loop with double buffering.  K is a multiple of BK.
__device__ void mma_k_loop(Tile &T, Loader &ld, int K, int wm, int wn, f32x16_t (&acc)[2][2]) {
  const int nk = K / BK;
  ld.fetch(0);
  ld.store(T, 0);
  __syncthreads();
  for (int kk = 0; kk < nk; ++kk) {
    const int buf = kk & 1;
    if (kk + 1 < nk) ld.fetch((kk + 1) * BK);
    mma_slice(T, buf, wm, wn, acc);
    if (kk + 1 < nk) ld.store(T, buf ^ 1);
    __syncthreads();
  }
}

__device__ __forceinline__ void zero_acc(f32x16_t (&acc)[2][2]) {
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
}

// row (within the 128-row tile) of accumulator element r of block (i, .)
__device__ __forceinline__ int acc_row(int wm, int i, int r) {
  return wm * 64 + i * 32 + (r >> 2) * 8 + (lane_id() >> 5) * 4 + (r & 3);
}

// ------------------------------------------------------------------ plan
// plan layout (int32): [0] U, [1] total M tiles, [4 .. 4+E) uniq,
// off[E+1], mt_off[E+1] (first M tile of each unique expert), list[n].
// Assignments of one expert appear in the order the atomic scatter gives;
// each GEMM row is computed independently of its position, so y does not
// depend on that order.
__global__ __launch_bounds__(1024) void prefill_plan_kernel(const int32_t *__restrict__ ids,
                                                            int64_t n, int E,
                                                            int32_t *__restrict__ plan) {
  __shared__ int32_t cnt[kMaxExperts], uidx[kMaxExperts], fill[kMaxExperts];
  __shared__ int32_t s_off[kMaxExperts + 1];
  __shared__ int32_t wsum[16][3];
  int32_t *uniq = plan + 4;
  int32_t *off = uniq + E;
  int32_t *mt_off = off + E + 1;
  int32_t *list = mt_off + E + 1;
  const int tid = threadIdx.x, lane = lane_id(), wv = tid >> 6;
  for (int e = tid; e < E; e += 1024) {
    cnt[e] = 0;
    fill[e] = 0;
  }
  __syncthreads();
  for (int64_t i = tid; i < n; i += 1024) atomicAdd(&cnt[ids[i]], 1);
  __syncthreads();
  const int c = tid < E ? cnt[tid] : 0;
  int v[3] = {c > 0 ? 1 : 0, c, (c + BM - 1) / BM};
  int inc[3] = {v[0], v[1], v[2]};
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
#pragma unroll
    for (int q = 0; q < 3; ++q) {
      const int t = __shfl_up(inc[q], o);
      if (lane >= o) inc[q] += t;
    }
  }
  if (lane == kWave - 1)
    for (int q = 0; q < 3; ++q) wsum[wv][q] = inc[q];
  __syncthreads();
  int base[3] = {0, 0, 0};
  for (int k = 0; k < wv; ++k)
    for (int q = 0; q < 3; ++q) base[q] += wsum[k][q];
  const int ex_u = base[0] + inc[0] - v[0];
  const int ex_c = base[1] + inc[1] - v[1];
  const int ex_m = base[2] + inc[2] - v[2];
  if (tid < E) {
    uidx[tid] = ex_u;
    if (c > 0) {
      uniq[ex_u] = tid;
      off[ex_u] = ex_c;
      s_off[ex_u] = ex_c;
      mt_off[ex_u] = ex_m;
    }
  }
  if (tid == 1023) {
    const int U = base[0] + inc[0];
    plan[0] = U;
    plan[1] = base[2] + inc[2];
    off[U] = (int32_t)n;
    mt_off[U] = base[2] + inc[2];
  }
  __syncthreads();
  for (int64_t i = tid; i < n; i += 1024) {
    const int e = ids[i];
    const int pos = atomicAdd(&fill[e], 1);
    list[s_off[uidx[e]] + pos] = (int32_t)i;
  }
}

// Locate M tile `mt` of the batch: unique expert u (binary search over
// mt_off) and the first row of the tile within u's list.
__device__ __forceinline__ void locate_tile(const int32_t *mt_off, int U, int mt, int *u_out,
                                            int *row0) {
  int lo = 0, hi = U - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (mt_off[mid] <= mt)
      lo = mid;
    else
      hi = mid - 1;
  }
  *u_out = lo;
  *row0 = (mt - mt_off[lo]) * BM;
}

// ------------------------------------------------------------------ gate/up
// Tile (M tile of expert u, 64 channels c0..c0+63).  B rows interleave gate
// and up: rows [64g, 64g+32) = Wg[e, c0+32g ..], rows [64g+32, 64g+64) =
// Wu[e, c0+32g ..]; wave (wm, wn) then holds the gate and the up value of
// the same (row, channel) in acc[i][0] and acc[i][1] of the same lane.
__global__ __launch_bounds__(kThreads) void gateup_mma_kernel(
    const uint16_t *__restrict__ x, int H, const uint16_t *__restrict__ Wg,
    const uint16_t *__restrict__ Wu, int I, const int32_t *__restrict__ plan, int E, int k1,
    const float *__restrict__ w, uint16_t *__restrict__ abf) {
  __shared__ Tile T;
  const int n_nt = I / 64;
  const int mt = blockIdx.x / n_nt, nt = blockIdx.x - mt * n_nt;
  const int U = plan[0];
  if (mt >= plan[1]) return;
  const int32_t *uniq = plan + 4;
  const int32_t *off = uniq + E;
  const int32_t *mt_off = off + E + 1;
  const int32_t *list = mt_off + E + 1;
  int u, row0;
  locate_tile(mt_off, U, mt, &u, &row0);
  const int e = uniq[u];
  const int lb = off[u], n_e = off[u + 1] - lb;
  const int c0 = nt * 64;
  const int tid = threadIdx.x, wv = tid >> 6, wm = wv >> 1, wn = wv & 1;
  Loader ld;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int ch = tid * 2 + i;
    ld.r[i] = ch >> 2;
    ld.q[i] = ch & 3;
    const int m = min(row0 + ld.r[i], n_e - 1);
    ld.arow[i] = x + (int64_t)(list[lb + m] / k1) * H;
    const int g = ld.r[i] >> 6, within = ld.r[i] & 63;
    const int cc = c0 + g * 32 + (within & 31);
    ld.brow[i] = (within < 32 ? Wg : Wu) + ((int64_t)e * I + cc) * H;
  }
  f32x16_t acc[2][2];
  zero_acc(acc);
  mma_k_loop(T, ld, H, wm, wn, acc);
  const int c = c0 + wn * 32 + (lane_id() & 31);
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = row0 + acc_row(wm, i, r);
      if (m < n_e) {
        const int asg = list[lb + m];
        const float a = silu(acc[i][0][r]) * acc[i][1][r] * w[asg];
        abf[(int64_t)asg * I + c] = (uint16_t)f32_to_bf16_bits(a);
      }
    }
}

// ------------------------------------------------------------------ down
// Tile (M tile of expert u, 128 output rows h0..h0+127 of H):
// z[asg, h] = a[asg, :] . Wd[e, h, :], stored as bf16 (the layer's output is
// bf16; partials in bf16 halve the traffic of the slot combine).
__global__ __launch_bounds__(kThreads) void down_mma_kernel(
    const uint16_t *__restrict__ abf, int H, const uint16_t *__restrict__ Wd, int I,
    const int32_t *__restrict__ plan, int E, uint16_t *__restrict__ zbf) {
  __shared__ Tile T;
  const int n_nt = H / BN;
  const int mt = blockIdx.x / n_nt, nt = blockIdx.x - mt * n_nt;
  const int U = plan[0];
  if (mt >= plan[1]) return;
  const int32_t *uniq = plan + 4;
  const int32_t *off = uniq + E;
  const int32_t *mt_off = off + E + 1;
  const int32_t *list = mt_off + E + 1;
  int u, row0;
  locate_tile(mt_off, U, mt, &u, &row0);
  const int e = uniq[u];
  const int lb = off[u], n_e = off[u + 1] - lb;
  const int h0 = nt * BN;
  const int tid = threadIdx.x, wv = tid >> 6, wm = wv >> 1, wn = wv & 1;
  Loader ld;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int ch = tid * 2 + i;
    ld.r[i] = ch >> 2;
    ld.q[i] = ch & 3;
    const int m = min(row0 + ld.r[i], n_e - 1);
    ld.arow[i] = abf + (int64_t)list[lb + m] * I;
    ld.brow[i] = Wd + ((int64_t)e * H + h0 + ld.r[i]) * I;
  }
  f32x16_t acc[2][2];
  zero_acc(acc);
  mma_k_loop(T, ld, I, wm, wn, acc);
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = row0 + acc_row(wm, i, r);
      if (m < n_e) {
        const int asg = list[lb + m];
#pragma unroll
        for (int j = 0; j < 2; ++j)
          zbf[(int64_t)asg * H + h0 + wn * 64 + j * 32 + (lane_id() & 31)] =
              (uint16_t)f32_to_bf16_bits(acc[i][j][r]);
      }
    }
}

// ------------------------------------------------------------------ router
// fp32 router weights as three bf16 terms, Wr = W1 + W2 + W3 with
// W1 = bf16(Wr), W2 = bf16(Wr - W1), W3 = bf16(Wr - W1 - W2): 24 significant
// bits, i.e. the fp32 value (up to the last bit's rounding).  x is bf16, so
// every product is exact in fp32 and logits = x W1^T + x W2^T + x W3^T with
// fp32 accumulation.
__global__ void split_router_kernel(const float *__restrict__ Wr, int64_t n,
                                    uint16_t *__restrict__ w3) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const float v = Wr[i];
  const uint32_t b1 = f32_to_bf16_bits(v);
  const float r1 = v - __uint_as_float(b1 << 16);
  const uint32_t b2 = f32_to_bf16_bits(r1);
  const float r2 = r1 - __uint_as_float(b2 << 16);
  const uint32_t b3 = f32_to_bf16_bits(r2);
  w3[i] = (uint16_t)b1;
  w3[n + i] = (uint16_t)b2;
  w3[2 * n + i] = (uint16_t)b3;
}

// Tile (128 tokens, 128 experts): the three terms are three K passes into
// one accumulator.  Experts beyond E read a valid row and are not stored.
__global__ __launch_bounds__(kThreads) void router_mma_kernel(
    const uint16_t *__restrict__ x, int64_t T, int H, const uint16_t *__restrict__ w3,
    const float *__restrict__ br, int E, float *__restrict__ logits,
    float *__restrict__ logits2) {
  __shared__ Tile Tl;
  const int n_nt = (E + BN - 1) / BN;
  const int64_t mt = blockIdx.x / n_nt;
  const int nt = (int)(blockIdx.x - mt * n_nt);
  const int tid = threadIdx.x, wv = tid >> 6, wm = wv >> 1, wn = wv & 1;
  const int64_t t0 = mt * BM;
  const int e0 = nt * BN;
  f32x16_t acc[2][2];
  zero_acc(acc);
  for (int term = 0; term < 3; ++term) {
    Loader ld;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int ch = tid * 2 + i;
      ld.r[i] = ch >> 2;
      ld.q[i] = ch & 3;
      const int64_t t = min<int64_t>(t0 + ld.r[i], T - 1);
      ld.arow[i] = x + t * H;
      const int e = min(e0 + ld.r[i], E - 1);
      ld.brow[i] = w3 + (int64_t)term * E * H + (int64_t)e * H;
    }
    mma_k_loop(Tl, ld, H, wm, wn, acc);
  }
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int64_t t = t0 + acc_row(wm, i, r);
      if (t < T) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int e = e0 + wn * 64 + j * 32 + (lane_id() & 31);
          if (e < E) {
            const float v = acc[i][j][r] + (br ? br[e] : 0.0f);
            logits[t * E + e] = v;
            if (logits2) logits2[t * E + e] = v;
          }
        }
      }
    }
}

}  // namespace pf

bool prefill_supported(int H, int I, bool bf16) {
  return bf16 && H % pf::BN == 0 && I % 64 == 0 && H % pf::BK == 0 && I % pf::BK == 0;
}

size_t prefill_plan_words(int64_t n, int E) { return 4 + 3 * (size_t)E + 2 + (size_t)n; }

hipError_t launch_split_router(const float *Wr, int E, int H, uint16_t *w3, hipStream_t s) {
  const int64_t n = (int64_t)E * H;
  pf::split_router_kernel<<<dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s>>>(Wr, n, w3);
  return hipGetLastError();
}

hipError_t launch_router_mma(const uint16_t *x, int64_t T, int H, const uint16_t *w3,
                             const float *br, int E, float *logits, float *logits2,
                             hipStream_t s) {
  const int64_t tiles = ((T + pf::BM - 1) / pf::BM) * ((E + pf::BN - 1) / pf::BN);
  pf::router_mma_kernel<<<dim3((unsigned)tiles), dim3(pf::kThreads), 0, s>>>(x, T, H, w3, br, E,
                                                                             logits, logits2);
  return hipGetLastError();
}

hipError_t launch_prefill_plan(const int32_t *ids, int64_t n, int E, int32_t *plan,
                               hipStream_t s) {
  pf::prefill_plan_kernel<<<1, 1024, 0, s>>>(ids, n, E, plan);
  return hipGetLastError();
}

// upper bound of the M tiles of a batch: one partial tile per expert
static int64_t max_mtiles(int64_t n, int E) {
  const int64_t u = n < E ? n : E;
  return (n + pf::BM - 1) / pf::BM + u;
}

hipError_t launch_gateup_mma(const uint16_t *x, int H, const uint16_t *Wg, const uint16_t *Wu,
                             int I, const int32_t *plan, int E, int64_t n, int k1, const float *w,
                             uint16_t *abf, hipStream_t s) {
  const int64_t grid = max_mtiles(n, E) * (I / 64);
  pf::gateup_mma_kernel<<<dim3((unsigned)grid), dim3(pf::kThreads), 0, s>>>(x, H, Wg, Wu, I, plan,
                                                                            E, k1, w, abf);
  return hipGetLastError();
}

hipError_t launch_down_mma(const uint16_t *abf, int H, const uint16_t *Wd, int I,
                           const int32_t *plan, int E, int64_t n, uint16_t *zbf, hipStream_t s) {
  const int64_t grid = max_mtiles(n, E) * (H / pf::BN);
  pf::down_mma_kernel<<<dim3((unsigned)grid), dim3(pf::kThreads), 0, s>>>(abf, H, Wd, I, plan, E,
                                                                          zbf);
  return hipGetLastError();
}

// y[t, h] = sum over the token's k1 slots of z[t*k1 + r, h] (bf16 partials,
// fp32 sum in slot order); 8 outputs per thread with 16-byte accesses.
__global__ __launch_bounds__(256) void combine_bf16_kernel(const uint16_t *__restrict__ zbf,
                                                           int64_t T, int H, int k1,
                                                           uint16_t *__restrict__ y) {
  const int64_t i8 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8;
  if (i8 >= T * H) return;
  const int64_t t = i8 / H, h = i8 - t * H;
  float s[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) s[k] = 0.0f;
  for (int r = 0; r < k1; ++r) {
    float v[8];
    Elem<bf16_t>::widen(ld16(zbf + (t * k1 + r) * H + h), v);
#pragma unroll
    for (int k = 0; k < 8; ++k) s[k] = s[k] + v[k];
  }
  uint4 o;
  o.x = f32_to_bf16_bits(s[0]) | (f32_to_bf16_bits(s[1]) << 16);
  o.y = f32_to_bf16_bits(s[2]) | (f32_to_bf16_bits(s[3]) << 16);
  o.z = f32_to_bf16_bits(s[4]) | (f32_to_bf16_bits(s[5]) << 16);
  o.w = f32_to_bf16_bits(s[6]) | (f32_to_bf16_bits(s[7]) << 16);
  *reinterpret_cast<uint4 *>(y + i8) = o;
}

hipError_t launch_combine_bf16(const uint16_t *zbf, int64_t T, int H, int k1, uint16_t *y,
                               hipStream_t s) {
  const int64_t n8 = T * H / 8;
  combine_bf16_kernel<<<dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, s>>>(zbf, T, H, k1, y);
  return hipGetLastError();
}

}  // namespace moe
