// v1_fp32.hip -- DIFF V1 forward in fp32 on the vector ALUs.
//
// Computes the same function as the bf16 MFMA kernel ("Differential
// Transformer V2" article, DiffAttnV1; subln and output scale from the
// nanoGPT issue "How best to implement a differential transformer?",
// Wilsontomass's module) with fp32 operands throughout, for callers that
// need fp32 accuracy.  gfx950 has no fp32-input MFMA fast enough to matter
// at these sizes, so this path is a plain LDS-tiled kernel:
//   * a workgroup of 256 threads owns 32 query rows of one differential
//     head and walks 32-key tiles up to the diagonal;
//   * scores: each (map, row) is handled by 4 lanes, 8 keys each; standard
//     online softmax (exact running max) in registers;
//   * P.V: each row is handled by 8 lanes, 2d/8 output columns each, for
//     both maps, reading P and V from LDS;
//   * epilogue: A1V/l1 - lam A2V/l2, RMSNorm over 2d (eps 1e-5) and the
//     (1 - lambda_init) scale, reduced across the row's 8 lanes.
#include <math.h>

#include "kernels.hpp"

namespace da {
namespace {

constexpr int kRows = 32;
constexpr int kKeys = 32;

template <int D>
struct F32Smem {
  static constexpr int QR = D + 1;       // odd row strides: conflict-free columns
  static constexpr int VR = 2 * D + 1;
  static constexpr int PR = kKeys + 1;
  float q[2][kRows * QR];
  float k[2][kKeys * QR];
  float v[kKeys * VR];
  float p[2][kRows * PR];
  float alpha[2][kRows];
  float l[2][kRows];
};

template <int D>
__global__ void __launch_bounds__(256) v1_fp32_kernel(const V1F32Args a) {
  constexpr int DV = 2 * D;
  constexpr int CPT = DV / 8;  // output columns per thread in the P.V phase
  using S = F32Smem<D>;
  __shared__ S sm;

  const int tid = threadIdx.x;
  const int logical = xcd_logical_id(blockIdx.x, a.B * a.H * a.tiles);
  const int unit = logical / a.tiles;
  const int tile = a.tiles - 1 - logical % a.tiles;
  const int b = unit / a.H, h = unit % a.H;
  const int T = a.T;
  const int i0 = tile * kRows;

  const float* qp[2] = {(const float*)a.q1.p + b * a.q1.sb + h * a.q1.sh,
                        (const float*)a.q2.p + b * a.q2.sb + h * a.q2.sh};
  const int64_t qst[2] = {a.q1.st, a.q2.st};
  const float* kp[2] = {(const float*)a.k1.p + b * a.k1.sb + h * a.k1.sh,
                        (const float*)a.k2.p + b * a.k2.sb + h * a.k2.sh};
  const int64_t kst[2] = {a.k1.st, a.k2.st};
  const float* vp = (const float*)a.v.p + b * a.v.sb + h * a.v.sh;

  // lambda = exp(lq1.lk1) - exp(lq2.lk2) + lambda_init (every wave computes it)
  float lam;
  {
    float pa = 0.f, pb = 0.f;
    for (int c = tid & 63; c < D; c += 64) {
      pa += a.lq1[c] * a.lk1[c];
      pb += a.lq2[c] * a.lk2[c];
    }
    lam = expf(wave_sum(pa)) - expf(wave_sum(pb)) + a.lam_init;
  }

  // Q tiles -> LDS
  for (int e = tid; e < 2 * kRows * (D / 4); e += 256) {
    const int m = e / (kRows * (D / 4)), rem = e % (kRows * (D / 4));
    const int r = rem / (D / 4), c4 = (rem % (D / 4)) * 4;
    const int row = i0 + r;
    float4 x = row < T ? *(const float4*)(qp[m] + (int64_t)row * qst[m] + c4) : make_float4(0, 0, 0, 0);
    float* d = &sm.q[m][r * S::QR + c4];
    d[0] = x.x, d[1] = x.y, d[2] = x.z, d[3] = x.w;
  }

  // score-phase role: (map, row, key group)
  const int sm_m = tid >> 7, sm_r = (tid >> 2) & 31, sm_kg = tid & 3;
  float m_run = -INFINITY, l_run = 0.f;
  // P.V-phase role: (row, column group)
  const int pv_r = tid >> 3, pv_cg = tid & 7;
  float acc[2][CPT];
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int c = 0; c < CPT; ++c) acc[m][c] = 0.f;

  const float sl2 = a.sl2;
  const int kend = min(T, i0 + kRows);
  for (int j0 = 0; j0 < kend; j0 += kKeys) {
    __syncthreads();  // previous tile fully consumed
    for (int e = tid; e < 2 * kKeys * (D / 4); e += 256) {
      const int m = e / (kKeys * (D / 4)), rem = e % (kKeys * (D / 4));
      const int r = rem / (D / 4), c4 = (rem % (D / 4)) * 4;
      const int key = j0 + r;
      float4 x = key < T ? *(const float4*)(kp[m] + (int64_t)key * kst[m] + c4) : make_float4(0, 0, 0, 0);
      float* d = &sm.k[m][r * S::QR + c4];
      d[0] = x.x, d[1] = x.y, d[2] = x.z, d[3] = x.w;
    }
    for (int e = tid; e < kKeys * (DV / 4); e += 256) {
      const int r = e / (DV / 4), c4 = (e % (DV / 4)) * 4;
      const int key = j0 + r;
      float4 x = key < T ? *(const float4*)(vp + (int64_t)key * a.v.st + c4) : make_float4(0, 0, 0, 0);
      float* d = &sm.v[r * S::VR + c4];
      d[0] = x.x, d[1] = x.y, d[2] = x.z, d[3] = x.w;
    }
    __syncthreads();

    // scores for (sm_m, sm_r) over keys sm_kg + 4*jj
    {
      const float* qr = &sm.q[sm_m][sm_r * S::QR];
      float s[8];
      float mx = -INFINITY;
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const int kk = sm_kg + 4 * jj;
        const float* kr = &sm.k[sm_m][kk * S::QR];
        float dot = 0.f;
#pragma unroll 8
        for (int c = 0; c < D; ++c) dot = fmaf(qr[c], kr[c], dot);
        s[jj] = (j0 + kk > i0 + sm_r) ? -INFINITY : dot * sl2;
        mx = fmaxf(mx, s[jj]);
      }
      mx = fmaxf(mx, __shfl_xor(mx, 1, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 2, 64));
      const float m_new = fmaxf(m_run, mx);  // finite: key j0 <= row always visible
      const float al = exp2f(m_run - m_new);
      float ps = 0.f;
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const float p = exp2f(s[jj] - m_new);
        ps += p;
        sm.p[sm_m][sm_r * S::PR + sm_kg + 4 * jj] = p;
      }
      ps += __shfl_xor(ps, 1, 64);
      ps += __shfl_xor(ps, 2, 64);
      l_run = l_run * al + ps;
      m_run = m_new;
      if (sm_kg == 0) sm.alpha[sm_m][sm_r] = al;
    }
    __syncthreads();

    // P.V for row pv_r, columns pv_cg + 8*c
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const float al = sm.alpha[m][pv_r];
#pragma unroll
      for (int c = 0; c < CPT; ++c) acc[m][c] *= al;
      const float* pr = &sm.p[m][pv_r * S::PR];
      for (int j = 0; j < kKeys; ++j) {
        const float p = pr[j];
        const float* vr = &sm.v[j * S::VR + pv_cg];
#pragma unroll
        for (int c = 0; c < CPT; ++c) acc[m][c] = fmaf(p, vr[8 * c], acc[m][c]);
      }
    }
  }

  // off-by-one softmax: one more logit 0, i.e. 2^(0 - m) against the running max
  if (sm_kg == 0) sm.l[sm_m][sm_r] = l_run + (a.softmax1 ? exp2f(-m_run) : 0.f);
  __syncthreads();

  const int row = i0 + pv_r;
  const float inv0 = 1.f / sm.l[0][pv_r], inv1 = 1.f / sm.l[1][pv_r];
  float ss = 0.f;
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const float dv = acc[0][c] * inv0 - lam * (acc[1][c] * inv1);
    acc[0][c] = dv;
    ss = fmaf(dv, dv, ss);
  }
  ss += __shfl_xor(ss, 1, 64);
  ss += __shfl_xor(ss, 2, 64);
  ss += __shfl_xor(ss, 4, 64);
  const float post = (1.f - a.lam_init) / sqrtf(ss / (float)DV + 1e-5f);
  if (row < T) {
    float* dst = (float*)a.out.p + b * a.out.sb + (int64_t)row * a.out.st + h * a.out.sh;
#pragma unroll
    for (int c = 0; c < CPT; ++c) dst[pv_cg + 8 * c] = acc[0][c] * post;
  }
}

template <int D>
hipError_t launch(const V1F32Args& a, hipStream_t s) {
  const void* args[] = {&a};
  return hipLaunchKernel((const void*)v1_fp32_kernel<D>, dim3(a.B * a.H * a.tiles), dim3(256), (void**)args, 0,
                         s);
}

}  // namespace

hipError_t launch_v1_fp32(int d, const V1F32Args& a0, hipStream_t s) {
  V1F32Args a = a0;
  a.tiles = (a.T + kRows - 1) / kRows;
  if (d == 32) return launch<32>(a, s);
  if (d == 64) return launch<64>(a, s);
  if (d == 128) return launch<128>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace da
