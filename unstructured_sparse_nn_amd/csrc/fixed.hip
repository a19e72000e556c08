// fixed.hip -- fixed-pattern inference kernels, generated per weight matrix
// and compiled at run time with hipRTC (gfx950).
//
// The idea follows SparseRT ("SparseRT: Accelerating Unstructured Sparsity on
// GPUs for Deep Learning Inference", Abstract): when the sparsity pattern
// and the values are fixed for inference, a code generator can turn them
// into the instruction stream itself, so the product reads no indices and no
// values from memory, only the activations.  The layout chosen here is this
// library's, for CDNA4:
//   * node-major activations, X: K x B per image, Y: M x B per image (a 1x1
//     convolution over an NCHW image is exactly this, B = H*W);
//   * the rows are cut into waves -- runs of at most RMAX consecutive rows,
//     about WAVE_NNZ entries -- whose accumulators live in registers, and
//     the waves into bands of up to MAX_WAVES; workgroup (x, y, z) computes
//     band y for the 64 batch columns 64x.. (one per lane) of image z, so a
//     fully connected layer of any size fills the GPU even at one batch
//     tile, and a small one (a 1x1 convolution) stages its inputs once per
//     batch tile;
//   * the inputs are staged in LDS as fp32 in tiles of KT columns x 64 batch
//     columns (coalesced loads); a band stages only the tiles holding one of
//     its entries.  Per tile, a wave walks the columns of its entries in
//     order, reads each staged input once and feeds every entry of that
//     column with the value as an immediate operand (v_fmamk_f32);
//   * results are rounded once to the activation type and stored coalesced.
// Everything is in one kernel (one launch per forward); code size and
// compile time grow linearly with nnz (13-22 bytes of code per entry: one
// FMA, plus a staged-input read per column of a wave's rows).
#include <hip/hip_runtime.h>
#include <hip/hiprtc.h>

#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "../../include/snack.h"

struct snack_fixed {
  int32_t M, K;
  int64_t nnz;
  snack_dtype dtype;
  int32_t waves;       // waves per workgroup
  int32_t bands;       // workgroups per batch tile and image
  hipModule_t module;  // null when built with SNACK_FIXED_COMPILE_ONLY
  hipFunction_t fn;
  size_t code_bytes;
  std::string source;
  std::vector<char> code;  // the compiled code object
};

namespace {

constexpr int KT = 256;               // staged inputs per tile: KT x 64 fp32 = 64 KB of LDS
constexpr int RMAX = 32;              // rows (accumulators) per wave
constexpr int64_t WAVE_NNZ = 512;     // entries per wave, about
constexpr int MAX_WAVES = 16;         // waves per workgroup
constexpr int64_t MAX_NNZ = 1 << 23;  // entries baked into one handle
constexpr int32_t MAX_BANDS = 65535;  // workgroups along grid y

std::string f32_literal(float v) {
  char buf[64];
  std::snprintf(buf, sizeof(buf), "%af", (double)v);  // exact hexadecimal form
  return buf;
}

float value_of(const void* vals, snack_dtype dt, int64_t k) {
  if (dt == SNACK_F32) return ((const float*)vals)[k];
  const uint32_t bits = (uint32_t)((const uint16_t*)vals)[k] << 16;
  float f;
  std::memcpy(&f, &bits, 4);
  return f;
}

struct wave_rows {
  int32_t r0, r1;  // rows [r0, r1)
};

// Waves: runs of consecutive rows, closed at RMAX rows or once they hold
// WAVE_NNZ entries; bands: up to `waves` consecutive waves.
std::vector<wave_rows> cut_waves(const std::vector<int64_t>& ptr, int32_t M) {
  std::vector<wave_rows> w;
  int32_t r = 0;
  while (r < M) {
    const int32_t r0 = r;
    int64_t n = 0;
    while (r < M && r - r0 < RMAX && (r == r0 || n < WAVE_NNZ)) {
      n += ptr[r + 1] - ptr[r];
      ++r;
    }
    w.push_back({r0, r});
  }
  return w;
}

std::string generate(const int32_t* row, const int32_t* col, const void* vals, snack_dtype dt,
                     int32_t M, int32_t K, int64_t nnz, int32_t* waves_out,
                     int32_t* bands_out) {
  std::vector<int64_t> ptr(M + 1, 0);
  for (int64_t k = 0; k < nnz; ++k) ++ptr[row[k] + 1];
  for (int32_t r = 0; r < M; ++r) ptr[r + 1] += ptr[r];
  const std::vector<wave_rows> wr = cut_waves(ptr, M);
  const int G = (int)std::min<size_t>(MAX_WAVES, wr.size());
  const int32_t bands = (int32_t)((wr.size() + G - 1) / G);
  *waves_out = G;
  *bands_out = bands;
  const char* T = dt == SNACK_F32 ? "float" : "unsigned short";
  const int32_t ntiles = (K + KT - 1) / KT;
  std::string s;
  s.reserve((size_t)nnz * 40 + (size_t)bands * 2048 + 4096);
  s += "typedef unsigned short bf16;\n";
  s += "__device__ __forceinline__ float ld(const float* p) { return *p; }\n";
  s += "__device__ __forceinline__ float ld(const bf16* p) { return __uint_as_float(((unsigned)*p) << 16); }\n";
  s += "__device__ __forceinline__ void st(float* p, float v) { *p = v; }\n";
  // round to nearest even, NaN kept quiet; branch-free
  s += "__device__ __forceinline__ void st(bf16* p, float v) {\n"
       "  const unsigned u = __float_as_uint(v);\n"
       "  const unsigned r = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;\n"
       "  *p = (bf16)(((u & 0x7FFFFFFFu) > 0x7F800000u) ? ((u >> 16) | 0x40u) : r);\n}\n";
  // the staged inputs: one LDS array for the workgroup, at file scope so
  // that every band function addresses it as LDS
  s += "__shared__ float xs[" + std::to_string(KT) + " * 64];\n";
  // inputs c0 .. c0+n-1 of the 64 batch columns, one column of xs per lane
  s += std::string("__device__ __forceinline__ void stage(const ") + T +
       "* Xi, int c0, int n, int w, int lane, long long b, int B) {\n"
       "  for (int c = w; c < n; c += " + std::to_string(G) +
       ") xs[c * 64 + lane] = b < B ? ld(Xi + (long long)(c0 + c) * B + b) : 0.f;\n}\n";
  // one function per band (bounded size for the compiler), called by the
  // workgroups of that band
  const std::string Ts(T);
  std::vector<std::vector<std::pair<int32_t, float>>> bycol(K);  // per column: (acc, value)
  for (int32_t band = 0; band < bands; ++band) {
    const size_t w0 = (size_t)band * G, w1 = std::min(wr.size(), w0 + G);
    s += "__device__ __attribute__((noinline)) void band" + std::to_string(band) +
         "(const " + Ts + "* __restrict__ Xi, " + Ts +
         "* __restrict__ Yi, long long b, int B, int w, int lane) {\n";
    int32_t rmax = 0;
    for (size_t wi = w0; wi < w1; ++wi) rmax = std::max(rmax, wr[wi].r1 - wr[wi].r0);
    for (int i = 0; i < rmax; ++i) s += "  float a" + std::to_string(i) + " = 0.f;\n";
    for (int32_t t = 0; t < ntiles; ++t) {
      const int32_t c0 = t * KT, c1 = std::min(K, c0 + KT);
      // does any entry of the band lie in this tile?  (rows are sorted by column)
      bool any = false;
      for (int32_t r = wr[w0].r0; r < wr[w1 - 1].r1 && !any; ++r) {
        const int32_t* lo = col + ptr[r];
        const int32_t* hi = col + ptr[r + 1];
        const int32_t* it = std::lower_bound(lo, hi, c0);
        any = it != hi && *it < c1;
      }
      if (!any) continue;
      s += "  stage(Xi, " + std::to_string(c0) + ", " + std::to_string(c1 - c0) +
           ", w, lane, b, B);\n  __syncthreads();\n  switch (w) {\n";
      for (size_t wi = w0; wi < w1; ++wi) {
        std::vector<int32_t> cols;
        for (int32_t r = wr[wi].r0; r < wr[wi].r1; ++r) {
          const int32_t* lo = col + ptr[r];
          const int32_t* hi = col + ptr[r + 1];
          for (const int32_t* it = std::lower_bound(lo, hi, c0); it != hi && *it < c1; ++it) {
            const int32_t c = *it;
            if (bycol[c].empty()) cols.push_back(c);
            bycol[c].push_back({r - wr[wi].r0, value_of(vals, dt, it - col)});
          }
        }
        if (cols.empty()) continue;
        std::sort(cols.begin(), cols.end());
        // columns in order: each staged input is read once and feeds every
        // entry of its column; the compiler pairs reads (ds_read2st64) and
        // schedules them ahead of the FMAs
        s += "  case " + std::to_string(wi - w0) + ":\n";
        for (size_t j = 0; j < cols.size(); ++j) {
          s += "    { const float x = xs[" + std::to_string(cols[j] - c0) + " * 64 + lane];";
          for (const auto& e : bycol[cols[j]])
            s += " a" + std::to_string(e.first) + " = __builtin_fmaf(" + f32_literal(e.second) +
                 ", x, a" + std::to_string(e.first) + ");";
          s += " }\n";
          bycol[cols[j]].clear();
        }
        s += "    break;\n";
      }
      s += "  }\n  __syncthreads();\n";
    }
    s += "  if (b < B) switch (w) {\n";
    for (size_t wi = w0; wi < w1; ++wi) {
      s += "  case " + std::to_string(wi - w0) + ":";
      for (int32_t r = wr[wi].r0; r < wr[wi].r1; ++r)
        s += " st(Yi + " + std::to_string(r) + "LL * B + b, a" + std::to_string(r - wr[wi].r0) +
             ");";
      s += " break;\n";
    }
    s += "  }\n}\n";
  }
  s += "extern \"C\" __global__ __launch_bounds__(" + std::to_string(64 * G) +
       ") void snk_fixed(const " + Ts + "* __restrict__ X, " + Ts +
       "* __restrict__ Y, int B, long long x_img, long long y_img) {\n";
  // the wave index, uniform over the wave: a scalar branch per wave
  s += "  const int lane = threadIdx.x & 63;\n";
  s += "  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);\n";
  s += "  const long long b = (long long)blockIdx.x * 64 + lane;\n";
  s += "  const " + Ts + "* Xi = X + (long long)blockIdx.z * x_img;\n";
  s += "  " + Ts + "* Yi = Y + (long long)blockIdx.z * y_img;\n";
  s += "  switch (blockIdx.y) {\n";
  for (int32_t band = 0; band < bands; ++band)
    s += "  case " + std::to_string(band) + ": band" + std::to_string(band) +
         "(Xi, Yi, b, B, w, lane); break;\n";
  s += "  }\n}\n";
  return s;
}

// The generated kernels target the MI355X only.
const char* offload_arch() { return "gfx950"; }

}  // namespace

extern "C" {

snack_status snack_fixed_build(const int32_t* row, const int32_t* col, const void* vals,
                               snack_dtype dtype, int32_t M, int32_t K, int64_t nnz,
                               uint32_t flags, snack_fixed** out) {
  if (!out) return SNACK_E_NULL;
  *out = nullptr;
  if (dtype != SNACK_F32 && dtype != SNACK_BF16) return SNACK_E_DTYPE;
  if (flags & ~(uint32_t)SNACK_FIXED_COMPILE_ONLY) return SNACK_E_LAYOUT;
  if (M < 1 || K < 1 || nnz < 0 || nnz > MAX_NNZ || (double)nnz > (double)M * K)
    return SNACK_E_SHAPE;
  if (nnz > 0 && (!row || !col || !vals)) return SNACK_E_NULL;
  int64_t prev = -1;
  for (int64_t k = 0; k < nnz; ++k) {
    if (row[k] < 0 || row[k] >= M || col[k] < 0 || col[k] >= K) return SNACK_E_COO_RANGE;
    const int64_t l = (int64_t)row[k] * K + col[k];
    if (l <= prev) return SNACK_E_COO_ORDER;
    prev = l;
  }
  snack_fixed* f = new snack_fixed();
  f->M = M;
  f->K = K;
  f->nnz = nnz;
  f->dtype = dtype;
  f->module = nullptr;
  f->fn = nullptr;
  f->source = generate(row, col, vals, dtype, M, K, nnz, &f->waves, &f->bands);
  if (f->bands > MAX_BANDS) {  // the launch's grid y
    delete f;
    return SNACK_E_SHAPE;
  }
  hiprtcProgram prog;
  if (hiprtcCreateProgram(&prog, f->source.c_str(), "snk_fixed.hip", 0, nullptr, nullptr) !=
      HIPRTC_SUCCESS) {
    delete f;
    return SNACK_E_HIP;
  }
  const std::string arch = std::string("--offload-arch=") + offload_arch();
  const char* opts[] = {arch.c_str(), "-O3", "-Xclang", "-target-feature", "-Xclang",
                        "-packed-fp32-ops"};
  const hiprtcResult cr = hiprtcCompileProgram(prog, 6, opts);
  size_t code_size = 0;
  std::vector<char> code;
  if (cr == HIPRTC_SUCCESS && hiprtcGetCodeSize(prog, &code_size) == HIPRTC_SUCCESS) {
    code.resize(code_size);
    if (hiprtcGetCode(prog, code.data()) != HIPRTC_SUCCESS) code_size = 0;
  }
  hiprtcDestroyProgram(&prog);
  if (cr != HIPRTC_SUCCESS || code_size == 0) {
    delete f;
    return SNACK_E_HIP;
  }
  f->code_bytes = code_size;
  f->code = code;
  if (!(flags & SNACK_FIXED_COMPILE_ONLY)) {
    if (hipModuleLoadData(&f->module, code.data()) != hipSuccess ||
        hipModuleGetFunction(&f->fn, f->module, "snk_fixed") != hipSuccess) {
      if (f->module) hipModuleUnload(f->module);
      delete f;
      return SNACK_E_HIP;
    }
  }
  *out = f;
  return SNACK_OK;
}

snack_status snack_fixed_fwd(const snack_fixed* f, const void* X, int32_t B, int32_t images,
                             void* Y, void* stream) {
  if (!f) return SNACK_E_NULL;
  if (B < 0 || images < 0) return SNACK_E_SHAPE;
  if (!f->fn) return SNACK_E_NOT_PREPARED;
  if (B == 0 || images == 0) return SNACK_OK;
  if (!X || !Y) return SNACK_E_NULL;
  int32_t Bi = B;
  long long x_img = (long long)f->K * B, y_img = (long long)f->M * B;
  void* args[] = {(void*)&X, (void*)&Y, (void*)&Bi, (void*)&x_img, (void*)&y_img};
  const int64_t gx = ((int64_t)B + 63) / 64;
  if (gx > INT32_MAX || images > 65535) return SNACK_E_SHAPE;
  if (hipModuleLaunchKernel(f->fn, (unsigned)gx, (unsigned)f->bands, (unsigned)images,
                            64 * f->waves, 1, 1, 0, (hipStream_t)stream, args,
                            nullptr) != hipSuccess)
    return SNACK_E_HIP;
  return SNACK_OK;
}

snack_status snack_fixed_info(const snack_fixed* f, int32_t* waves, int32_t* bands,
                              size_t* code_bytes, size_t* source_bytes) {
  if (!f) return SNACK_E_NULL;
  if (waves) *waves = f->waves;
  if (bands) *bands = f->bands;
  if (code_bytes) *code_bytes = f->code_bytes;
  if (source_bytes) *source_bytes = f->source.size();
  return SNACK_OK;
}

const void* snack_fixed_code(const snack_fixed* f, size_t* bytes) {
  if (!f) return nullptr;
  if (bytes) *bytes = f->code.size();
  return f->code.data();
}

void snack_fixed_free(snack_fixed* f) {
  if (!f) return;
  if (f->module) hipModuleUnload(f->module);
  delete f;
}

}  // extern "C"
