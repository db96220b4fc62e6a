// GPU-side partial attention over the resident selected blocks, A_gpu = GPUATTN(Q, B_gpu),
// and its FlashAttention-style merge with the host partials, A = MERGE(A_gpu, A_cpu)
// [ScoutAttention, arXiv:2603.27138, HTML Sec. 3.2; Algorithm 1].
//
// Work split.  A workgroup of 4 waves takes one (sequence, KV head) pair and a chunk of its
// selected resident blocks; each wave walks its share of the chunk 32 tokens at a time (one
// block of 32, or two blocks of 16) and keeps an online softmax for the G query heads of
// the group.  The waves are combined in LDS and the workgroup writes one un-normalised
// partial (o, m, l) per head; the reduce kernel combines a pair's chunk partials (and the
// host partial) per query head.  Chunking gives thousands of workgroups even for a few
// hundred pairs, which keeps all 256 CUs streaming.
//
// bf16 path, per 32-token step of a wave:
//   * K (32 x d) is loaded straight into MFMA A-operand registers: lane l holds token
//     l % 16 of a 16-token tile and 8 consecutive channels (16 bytes), so one load
//     instruction reads 16 token rows of 64 contiguous bytes each.
//   * S^T = K Q^T on v_mfma_f32_16x16x32_bf16.  Q's columns are the G heads split into a
//     bf16 high part (columns 0..7) and a bf16 low part q - hi (columns 8..15); adding the
//     two results recovers q . k to about 2^-17 relative, so the float32 query keeps its
//     precision while K stays bf16.
//   * the softmax runs on the MFMA output layout (lane l: head l % 8, four tokens) with
//     cross-lane shuffles; p is passed through a 1 KiB LDS slab to the PV layout.
//   * O += P V on the vector ALU: lane l owns 8 channels of every 4th (d = 128) token row,
//     V read with 16-byte loads that cover whole rows.
// float32 path (small fp32 workloads): K and V staged through LDS, plain per-lane dot
// products; same chunk partials.
//
// Internal log2 domain: logits are scaled by scale * log2(e) and exponentiated with exp2;
// m is reported in natural-log units.
#include <hip/hip_ext.h>

#include "common.hpp"
#include "kernels.hpp"

namespace sa {
namespace {

constexpr int kAttnWaves = 4;
constexpr int kStep = 32;  // tokens per wave step
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Partials of chunk c of pair p, head g: o at part_o[((p * nchunks + c) * G + g) * D],
// (m_log2, l) at part_ml[((p * nchunks + c) * G + g) * 2].
struct Partials {
  float* o;
  float* ml;
};

__device__ __forceinline__ Partials partial_ptrs(float* base, int pairs, int nchunks, int G,
                                                 int D) {
  Partials p;
  p.o = base;
  p.ml = base + (size_t)pairs * nchunks * G * D;
  return p;
}

template <int D, int BS, int G>
__global__ __launch_bounds__(256, 2) void attn_bf16_kernel(
    const float* __restrict__ q, const uint16_t* __restrict__ k_pool,
    const uint16_t* __restrict__ v_pool, const int32_t* __restrict__ table,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ gpu_blocks,
    const int32_t* __restrict__ n_gpu, int list_stride, int Hkv, int max_blocks,
    float scale_log2, int chunk_blocks, int nchunks, int pairs, float* __restrict__ part_base) {
  constexpr int KS = D / 32;          // MFMA k-steps over the head dimension
  constexpr int SPB = kStep / BS;     // blocks per step (1 or 2)
  constexpr int VLPR = D / 8;         // lanes per V row
  constexpr int VTPI = kWave / VLPR;  // V rows per load instruction
  constexpr int VJ = kStep / VTPI;    // V loads per lane per step

  __shared__ float p_lds[kAttnWaves][kStep][8];
  __shared__ float a_lds[kAttnWaves][8];
  __shared__ float o_red[kAttnWaves][G][D];
  __shared__ float ml_red[kAttnWaves][G][2];

  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
  const int pair = blockIdx.y;
  const int chunk = blockIdx.x;
  const int ng = n_gpu[pair];
  const int e_begin = chunk * chunk_blocks;
  if (e_begin >= ng) return;  // the reduce kernel reads only non-empty chunks
  const int e_end = min(ng, e_begin + chunk_blocks);
  const int s = pair / Hkv, h = pair % Hkv;
  const int len = seq_lens[s];
  const int32_t* list = gpu_blocks + (size_t)pair * list_stride;
  const int32_t* trow = table + (size_t)pair * max_blocks;

  const int c16 = lane % 16;   // MFMA column (head / hi-lo) and row-in-tile
  const int kq = lane / 16;    // MFMA k-group
  const int hcol = c16 & 7;    // head of this MFMA column

  // Q^T as the MFMA B operand: column c < 8 = bf16(q_c), column c >= 8 = bf16(q_c - hi)
  bf16x8 qb[KS];
  {
    const bool live = hcol < G;
    const float* qrow = q + ((size_t)s * Hkv * G + (size_t)h * G + (live ? hcol : 0)) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      uint32_t w[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t half[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const float v = live ? qrow[32 * ks + 8 * kq + 2 * i + j] : 0.f;
          const uint32_t hi = f32_to_bf16_rne(v);
          half[j] = c16 < 8 ? hi : f32_to_bf16_rne(v - __uint_as_float(hi << 16));
        }
        w[i] = half[0] | (half[1] << 16);
      }
      qb[ks] = __builtin_bit_cast(bf16x8, make_uint4(w[0], w[1], w[2], w[3]));
    }
  }

  float m_run = -INFINITY;   // per head hcol (log2 units), uniform over the head's lanes
  float l_lane = 0.f;        // this lane's share of l for head hcol
  float o_acc[G][8];
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int i = 0; i < 8; ++i) o_acc[g][i] = 0.f;

  const int vcg = lane % VLPR, vts = lane / VLPR;
  const int nsteps = (e_end - e_begin + SPB - 1) / SPB;
  for (int step = wave; step < nsteps; step += kAttnWaves) {
    // blocks of this step
    int page[SPB], nval[SPB];
#pragma unroll
    for (int j = 0; j < SPB; ++j) {
      const int e = e_begin + step * SPB + j;
      if (e < e_end) {
        const int blk = list[e];
        page[j] = trow[blk];
        nval[j] = min(BS, len - blk * BS);
      } else {
        page[j] = -1;
        nval[j] = 0;
      }
    }
    // K into A-operand registers: tile tt covers step tokens 16tt .. 16tt+15
    uint4 kr[2][KS];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const int j = SPB == 1 ? 0 : tt;
      const int tok = SPB == 1 ? 16 * tt + c16 : c16;
      const bool ok = page[j] >= 0;
      const uint16_t* src = k_pool + ((size_t)(ok ? page[j] : 0) * BS + tok) * D + 8 * kq;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        kr[tt][ks] = ok ? *reinterpret_cast<const uint4*>(src + 32 * ks) : make_uint4(0, 0, 0, 0);
    }
    // V rows for the PV product: step token t = jj * VTPI + vts
    uint4 vr[VJ];
#pragma unroll
    for (int jj = 0; jj < VJ; ++jj) {
      const int t = jj * VTPI + vts;
      const int j = t / BS;
      const bool ok = (t % BS) < nval[j];  // masked rows are not read (p = 0 there)
      vr[jj] = ok ? *reinterpret_cast<const uint4*>(
                        v_pool + ((size_t)page[j] * BS + (t % BS)) * D + 8 * vcg)
                  : make_uint4(0, 0, 0, 0);
    }

    // S^T tiles: acc[tt][r] = logit of token 16tt + 4kq + r for MFMA column c16
    float sc[2][4];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kr[tt][ks]),
                                                      qb[ks], acc, 0, 0, 0);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float tot = acc[r] + __shfl_xor(acc[r], 8, kWave);  // hi + lo columns
        const int j = SPB == 1 ? 0 : tt;
        const int tin = SPB == 1 ? 16 * tt + 4 * kq + r : 4 * kq + r;  // token in block
        sc[tt][r] = tin < nval[j] ? tot * scale_log2 : -INFINITY;
      }
    }
    // online softmax for head hcol
    float mx = fmaxf(fmaxf(fmaxf(sc[0][0], sc[0][1]), fmaxf(sc[0][2], sc[0][3])),
                     fmaxf(fmaxf(sc[1][0], sc[1][1]), fmaxf(sc[1][2], sc[1][3])));
    mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
    mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
    const float m_new = fmaxf(m_run, mx);
    const bool none = m_new == -INFINITY;
    const float alpha = none ? 1.f : fast_exp2(m_run - m_new);
    float psum = 0.f;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = none ? 0.f : fast_exp2(sc[tt][r] - m_new);
        sc[tt][r] = p;
        psum += p;
      }
    l_lane = l_lane * alpha + psum;
    m_run = m_new;
    if (c16 < 8) {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int r = 0; r < 4; ++r) p_lds[wave][16 * tt + 4 * kq + r][c16] = sc[tt][r];
      if (kq == 0) a_lds[wave][c16] = alpha;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // O = alpha O + P V
    float al[8];
    *reinterpret_cast<float4*>(al) = *reinterpret_cast<const float4*>(&a_lds[wave][0]);
    *reinterpret_cast<float4*>(al + 4) = *reinterpret_cast<const float4*>(&a_lds[wave][4]);
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int i = 0; i < 8; ++i) o_acc[g][i] *= al[g];
#pragma unroll
    for (int jj = 0; jj < VJ; ++jj) {
      const int t = jj * VTPI + vts;
      float pv[8];
      *reinterpret_cast<float4*>(pv) = *reinterpret_cast<const float4*>(&p_lds[wave][t][0]);
      *reinterpret_cast<float4*>(pv + 4) = *reinterpret_cast<const float4*>(&p_lds[wave][t][4]);
      float v[8];
      bf16x8_to_f32(vr[jj], v);
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int i = 0; i < 8; ++i) o_acc[g][i] = fmaf(pv[g], v[i], o_acc[g][i]);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }

  // wave totals: l over the four k-groups, o over the VTPI token phases
  float l_w = l_lane + __shfl_xor(l_lane, 16, kWave);
  l_w += __shfl_xor(l_w, 32, kWave);
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float v = o_acc[g][i];
#pragma unroll
      for (int o = VLPR; o < kWave; o <<= 1) v += __shfl_xor(v, o, kWave);
      o_acc[g][i] = v;
    }
  if (vts == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      *reinterpret_cast<float4*>(&o_red[wave][g][8 * vcg]) =
          make_float4(o_acc[g][0], o_acc[g][1], o_acc[g][2], o_acc[g][3]);
      *reinterpret_cast<float4*>(&o_red[wave][g][8 * vcg + 4]) =
          make_float4(o_acc[g][4], o_acc[g][5], o_acc[g][6], o_acc[g][7]);
    }
  }
  if (lane < G) {  // lane g: c16 = g, kq = 0
    ml_red[wave][lane][0] = m_run;
    ml_red[wave][lane][1] = l_w;
  }
  __syncthreads();

  // combine the 4 waves and write this chunk's partial
  const Partials part = partial_ptrs(part_base, pairs, nchunks, G, D);
  const size_t slot = ((size_t)pair * nchunks + chunk) * G;
  for (int idx = threadIdx.x; idx < G * D; idx += blockDim.x) {
    const int g = idx / D, c = idx % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kAttnWaves; ++w) M = fmaxf(M, ml_red[w][g][0]);
    float acc = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kAttnWaves; ++w) {
        const float mw = ml_red[w][g][0];
        if (mw != -INFINITY) acc += fast_exp2(mw - M) * o_red[w][g][c];
      }
    }
    part.o[(slot + g) * D + c] = acc;
  }
  if (threadIdx.x < G) {
    const int g = threadIdx.x;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kAttnWaves; ++w) M = fmaxf(M, ml_red[w][g][0]);
    float L = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kAttnWaves; ++w) {
        const float mw = ml_red[w][g][0];
        if (mw != -INFINITY) L += fast_exp2(mw - M) * ml_red[w][g][1];
      }
    }
    part.ml[(slot + g) * 2 + 0] = M;
    part.ml[(slot + g) * 2 + 1] = L;
  }
}

// float32 KV: one wave per (pair, chunk); K and V blocks staged in LDS.
template <int D, int BS>
__global__ __launch_bounds__(64) void attn_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k_pool,
    const float* __restrict__ v_pool, const int32_t* __restrict__ table,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ gpu_blocks,
    const int32_t* __restrict__ n_gpu, int list_stride, int Hkv, int G, int max_blocks,
    float scale_log2, int chunk_blocks, int nchunks, int pairs, float* __restrict__ part_base) {
  constexpr int CPL = D / kWave;  // channels per lane (1 or 2)
  __shared__ float qs[8][D];
  __shared__ float ks[BS][D + 1];
  __shared__ float vs[BS][D];
  __shared__ float sc[8][BS];
  const int lane = threadIdx.x;
  const int pair = blockIdx.y, chunk = blockIdx.x;
  const int ng = n_gpu[pair];
  const int e_begin = chunk * chunk_blocks;
  if (e_begin >= ng) return;
  const int e_end = min(ng, e_begin + chunk_blocks);
  const int s = pair / Hkv, h = pair % Hkv;
  const int len = seq_lens[s];
  for (int i = lane; i < G * D; i += kWave)
    qs[i / D][i % D] = q[((size_t)s * Hkv * G + (size_t)h * G) * D + i];
  float m_run[8], l_run[8], o[8][CPL];
  for (int g = 0; g < 8; ++g) {
    m_run[g] = -INFINITY;
    l_run[g] = 0.f;
    for (int c = 0; c < CPL; ++c) o[g][c] = 0.f;
  }
  for (int e = e_begin; e < e_end; ++e) {
    const int blk = gpu_blocks[(size_t)pair * list_stride + e];
    const int page = table[(size_t)pair * max_blocks + blk];
    const int nval = min(BS, len - blk * BS);
    __syncthreads();
    for (int i = lane; i < BS * D; i += kWave) {
      ks[i / D][i % D] = k_pool[(size_t)page * BS * D + i];
      vs[i / D][i % D] = v_pool[(size_t)page * BS * D + i];
    }
    __syncthreads();
    for (int i = lane; i < G * BS; i += kWave) {
      const int g = i / BS, t = i % BS;
      float acc = 0.f;
      for (int c = 0; c < D; ++c) acc = fmaf(qs[g][c], ks[t][c], acc);
      sc[g][t] = t < nval ? acc * scale_log2 : -INFINITY;
    }
    __syncthreads();
    for (int g = 0; g < G; ++g) {
      float mx = -INFINITY;
      for (int t = 0; t < BS; ++t) mx = fmaxf(mx, sc[g][t]);
      const float m_new = fmaxf(m_run[g], mx);
      const float alpha = fast_exp2(m_run[g] - m_new);  // m_new is finite: nval >= 1
      float ps = 0.f;
      float acc[CPL];
      for (int c = 0; c < CPL; ++c) acc[c] = 0.f;
      for (int t = 0; t < BS; ++t) {
        const float p = fast_exp2(sc[g][t] - m_new);
        ps += p;
        for (int c = 0; c < CPL; ++c) acc[c] = fmaf(p, vs[t][lane + kWave * c], acc[c]);
      }
      l_run[g] = l_run[g] * alpha + ps;
      for (int c = 0; c < CPL; ++c) o[g][c] = o[g][c] * alpha + acc[c];
      m_run[g] = m_new;
    }
  }
  const Partials part = partial_ptrs(part_base, pairs, nchunks, G, D);
  const size_t slot = ((size_t)pair * nchunks + chunk) * G;
  for (int g = 0; g < G; ++g) {
    for (int c = 0; c < CPL; ++c) part.o[(slot + g) * D + lane + kWave * c] = o[g][c];
    if (lane == 0) {
      part.ml[(slot + g) * 2 + 0] = m_run[g];
      part.ml[(slot + g) * 2 + 1] = l_run[g];
    }
  }
}

// One wave per (sequence, query head) row: combine the pair's chunk partials and, when
// given, the host partial; write the normalised output.
template <int D>
__global__ __launch_bounds__(256) void reduce_kernel(
    const float* __restrict__ part_base, int pairs, int nchunks, int chunk_blocks, int G,
    int Hkv, int rows, const int32_t* __restrict__ n_gpu, const float* __restrict__ host_o,
    const float* __restrict__ host_m, const float* __restrict__ host_l,
    const int32_t* __restrict__ n_cpu, float* __restrict__ o, float* __restrict__ m,
    float* __restrict__ l) {
  constexpr int CPL = D / kWave;
  const int lane = threadIdx.x % kWave;
  const int row = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  if (row >= rows) return;
  const int Hq = Hkv * G;
  const int s = row / Hq, qh = row % Hq;
  const int pair = s * Hkv + qh / G, g = qh % G;
  const int nch = (n_gpu[pair] + chunk_blocks - 1) / chunk_blocks;
  const Partials part = partial_ptrs(const_cast<float*>(part_base), pairs, nchunks, G, D);
  const size_t slot0 = (size_t)pair * nchunks * G + g;

  float M = -INFINITY;
  for (int c = 0; c < nch; ++c) M = fmaxf(M, part.ml[(slot0 + (size_t)c * G) * 2]);
  bool use_host = host_o != nullptr && (n_cpu == nullptr || n_cpu[pair] > 0);
  float mh = -INFINITY, lh = 0.f;
  if (use_host) {
    mh = host_m[row] * kLog2e;
    lh = host_l[row];
    if (!(lh > 0.f) || mh == -INFINITY) use_host = false;
    else M = fmaxf(M, mh);
  }
  float acc[CPL], L = 0.f;
#pragma unroll
  for (int i = 0; i < CPL; ++i) acc[i] = 0.f;
  if (M != -INFINITY) {
    for (int c = 0; c < nch; ++c) {
      const size_t sl = slot0 + (size_t)c * G;
      const float mc = part.ml[sl * 2];
      if (mc == -INFINITY) continue;
      const float w = fast_exp2(mc - M);
      L += w * part.ml[sl * 2 + 1];
#pragma unroll
      for (int i = 0; i < CPL; ++i) acc[i] = fmaf(w, part.o[sl * D + lane + kWave * i], acc[i]);
    }
    if (use_host) {
      const float w = lh * fast_exp2(mh - M);
      L += w;
#pragma unroll
      for (int i = 0; i < CPL; ++i)
        acc[i] = fmaf(w, host_o[(size_t)row * D + lane + kWave * i], acc[i]);
    }
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
#pragma unroll
  for (int i = 0; i < CPL; ++i) o[(size_t)row * D + lane + kWave * i] = acc[i] * inv;
  if (lane == 0) {
    if (m) m[row] = M == -INFINITY ? -INFINITY : M * kLn2;
    if (l) l[row] = L;
  }
}

// Elementwise merge of two normalised partials, one wave per row.
__global__ __launch_bounds__(256) void merge_kernel(int rows, int d, const float* o_a,
                                                    const float* m_a, const float* l_a,
                                                    const float* o_b, const float* m_b,
                                                    const float* l_b, float* o, float* m,
                                                    float* l) {
  const int lane = threadIdx.x % kWave;
  const int row = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  if (row >= rows) return;
  const float ma = m_a[row], mb = m_b[row];
  const float la = l_a[row], lb = l_b[row];
  const float M = fmaxf(ma, mb);
  float wa = 0.f, wb = 0.f;
  if (M != -INFINITY) {
    if (ma != -INFINITY) wa = la * expf(ma - M);
    if (mb != -INFINITY) wb = lb * expf(mb - M);
  }
  const float L = wa + wb;
  const float inv = L > 0.f ? 1.f / L : 0.f;
  for (int c = lane; c < d; c += kWave) {
    const size_t i = (size_t)row * d + c;
    o[i] = (wa * o_a[i] + wb * o_b[i]) * inv;
  }
  // all lanes have read m_a / l_a before lane 0 overwrites them (outputs may alias a)
  __builtin_amdgcn_wave_barrier();
  if (lane == 0) {
    m[row] = L > 0.f ? M : -INFINITY;
    l[row] = L;
  }
}

template <int D, int BS>
hipError_t attn_bf16_g(const Shape& s, const AttnPlan& p, const float* q, const void* k,
                       const void* v, const int32_t* t, const int32_t* lens,
                       const int32_t* gb, const int32_t* ng, int stride, float sl2,
                       float* part, hipStream_t st, hipEvent_t e0, hipEvent_t e1) {
  const dim3 grid(p.nchunks, s.B * s.Hkv), block(kAttnWaves * kWave);
  const int pairs = s.B * s.Hkv;
  // hipExtLaunchKernelGGL records the (optional) events at the kernel's own start and end
#define SA_ATTN_CASE(GG)                                                                    \
  case GG:                                                                                  \
    hipExtLaunchKernelGGL((attn_bf16_kernel<D, BS, GG>), grid, block, 0, st, e0, e1, 0, q,  \
                          (const uint16_t*)k, (const uint16_t*)v, t, lens, gb, ng, stride,   \
                          s.Hkv, s.max_blocks, sl2, p.chunk_blocks, p.nchunks, pairs, part); \
    break;
  switch (s.G) {
    SA_ATTN_CASE(1) SA_ATTN_CASE(2) SA_ATTN_CASE(3) SA_ATTN_CASE(4)
    SA_ATTN_CASE(5) SA_ATTN_CASE(6) SA_ATTN_CASE(7) SA_ATTN_CASE(8)
    default: return hipErrorInvalidValue;
  }
#undef SA_ATTN_CASE
  return hipGetLastError();
}

template <int D, int BS>
hipError_t attn_f32(const Shape& s, const AttnPlan& p, const float* q, const void* k,
                    const void* v, const int32_t* t, const int32_t* lens, const int32_t* gb,
                    const int32_t* ng, int stride, float sl2, float* part, hipStream_t st,
                    hipEvent_t e0, hipEvent_t e1) {
  const dim3 grid(p.nchunks, s.B * s.Hkv);
  hipExtLaunchKernelGGL((attn_f32_kernel<D, BS>), grid, dim3(kWave), 0, st, e0, e1, 0, q,
                        (const float*)k, (const float*)v, t, lens, gb, ng, stride, s.Hkv, s.G,
                        s.max_blocks, sl2, p.chunk_blocks, p.nchunks, s.B * s.Hkv, part);
  return hipGetLastError();
}

}  // namespace

AttnPlan attn_plan(const Shape& s, int list_stride) {
  AttnPlan p;
  // bf16: 4 waves x 4 steps of 32 tokens; float32: a few blocks per single-wave group
  p.chunk_tokens = s.bf16 ? kAttnWaves * 4 * kStep : 4 * s.bs;
  p.chunk_blocks = p.chunk_tokens / s.bs;
  p.nchunks = (list_stride + p.chunk_blocks - 1) / p.chunk_blocks;
  p.ws_bytes = (size_t)s.B * s.Hkv * p.nchunks * s.G * (s.d + 2) * sizeof(float);
  return p;
}

hipError_t launch_attention(const Shape& s, const AttnPlan& plan, const float* q,
                            const void* k_pool, const void* v_pool,
                            const int32_t* block_table, const int32_t* seq_lens,
                            const int32_t* gpu_blocks, const int32_t* n_gpu, int list_stride,
                            float scale, float* partials, hipStream_t stream,
                            hipEvent_t ev_start, hipEvent_t ev_stop) {
  const float sl2 = scale * kLog2e;
#define SA_ARGS plan, q, k_pool, v_pool, block_table, seq_lens, gpu_blocks, n_gpu, \
                list_stride, sl2, partials, stream, ev_start, ev_stop
  if (s.bf16) {
    if (s.d == 128) return s.bs == 32 ? attn_bf16_g<128, 32>(s, SA_ARGS) : attn_bf16_g<128, 16>(s, SA_ARGS);
    return s.bs == 32 ? attn_bf16_g<64, 32>(s, SA_ARGS) : attn_bf16_g<64, 16>(s, SA_ARGS);
  }
  if (s.d == 128) return s.bs == 32 ? attn_f32<128, 32>(s, SA_ARGS) : attn_f32<128, 16>(s, SA_ARGS);
  return s.bs == 32 ? attn_f32<64, 32>(s, SA_ARGS) : attn_f32<64, 16>(s, SA_ARGS);
#undef SA_ARGS
}

hipError_t launch_reduce(const Shape& s, const AttnPlan& plan, const int32_t* n_gpu,
                         const float* partials, const float* host_o, const float* host_m,
                         const float* host_l, const int32_t* n_cpu, float* o, float* m,
                         float* l, hipStream_t stream) {
  const int rows = s.B * s.Hq;
  const dim3 grid((rows + 3) / 4), block(256);
  if (s.d == 128)
    hipLaunchKernelGGL(reduce_kernel<128>, grid, block, 0, stream, partials, s.B * s.Hkv,
                       plan.nchunks, plan.chunk_blocks, s.G, s.Hkv, rows, n_gpu, host_o,
                       host_m, host_l, n_cpu, o, m, l);
  else
    hipLaunchKernelGGL(reduce_kernel<64>, grid, block, 0, stream, partials, s.B * s.Hkv,
                       plan.nchunks, plan.chunk_blocks, s.G, s.Hkv, rows, n_gpu, host_o,
                       host_m, host_l, n_cpu, o, m, l);
  return hipGetLastError();
}

hipError_t launch_merge(int rows, int d, const float* o_a, const float* m_a, const float* l_a,
                        const float* o_b, const float* m_b, const float* l_b, float* o,
                        float* m, float* l, hipStream_t stream) {
  hipLaunchKernelGGL(merge_kernel, dim3((rows + 3) / 4), dim3(256), 0, stream, rows, d, o_a,
                     m_a, l_a, o_b, m_b, l_b, o, m, l);
  return hipGetLastError();
}

}  // namespace sa
