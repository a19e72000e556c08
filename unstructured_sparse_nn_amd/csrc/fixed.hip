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
//   * one workgroup covers 64 consecutive batch columns (one per lane); the
//     K input values of those columns are staged in LDS as fp32 with
//     coalesced loads;
//   * the rows are cut into R contiguous groups of about equal nnz, one per
//     wave; a wave walks its rows in chunks of at most CHUNK rows, and inside
//     a chunk column by column, so each staged input is read from LDS once
//     per chunk and feeds every entry of that column with the value as an
//     immediate operand (v_fmamk_f32); accumulators live in registers;
//   * results are rounded once to the activation type and stored coalesced.
#include <hip/hip_runtime.h>
#include <hip/hiprtc.h>

#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <string>
#include <vector>

#include "../../include/snack.h"

struct snack_fixed {
  int32_t M, K;
  int64_t nnz;
  snack_dtype dtype;
  int32_t groups;      // waves per workgroup
  hipModule_t module;  // null when built with SNACK_FIXED_COMPILE_ONLY
  hipFunction_t fn;
  size_t code_bytes;
  std::string source;
  std::vector<char> code;  // the compiled code object
};

namespace {

constexpr int CHUNK = 32;          // rows whose accumulators a wave keeps at once
constexpr int PIPE = 4;            // staged-input reads in flight ahead of the FMAs
constexpr int MAX_GROUPS = 16;     // waves per workgroup
constexpr int32_t MAX_K = 256;     // staged inputs: K x 64 fp32 <= 64 KB of LDS
constexpr int64_t MAX_NNZ = 65536; // entries baked into one kernel

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

// Row groups: contiguous row ranges of about nnz / groups entries each.
std::vector<int32_t> group_starts(const std::vector<int64_t>& ptr, int32_t M, int groups) {
  std::vector<int32_t> g(groups + 1, M);
  g[0] = 0;
  const int64_t nnz = ptr[M];
  int32_t r = 0;
  for (int i = 1; i < groups; ++i) {
    const int64_t target = nnz * i / groups;
    while (r < M && ptr[r] < target) ++r;
    g[i] = std::max(g[i - 1], r);
  }
  return g;
}

std::string generate(const int32_t* row, const int32_t* col, const void* vals, snack_dtype dt,
                     int32_t M, int32_t K, int64_t nnz, int groups) {
  std::vector<int64_t> ptr(M + 1, 0);
  for (int64_t k = 0; k < nnz; ++k) ++ptr[row[k] + 1];
  for (int32_t r = 0; r < M; ++r) ptr[r + 1] += ptr[r];
  const std::vector<int32_t> gs = group_starts(ptr, M, groups);
  const char* T = dt == SNACK_F32 ? "float" : "unsigned short";
  std::string s;
  s.reserve((size_t)nnz * 48 + 4096);
  s += "typedef unsigned short bf16;\n";
  s += "__device__ __forceinline__ float ld(const float* p) { return *p; }\n";
  s += "__device__ __forceinline__ float ld(const bf16* p) { return __uint_as_float(((unsigned)*p) << 16); }\n";
  s += "__device__ __forceinline__ void st(float* p, float v) { *p = v; }\n";
  // round to nearest even, NaN kept quiet; branch-free
  s += "__device__ __forceinline__ void st(bf16* p, float v) {\n"
       "  const unsigned u = __float_as_uint(v);\n"
       "  const unsigned r = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;\n"
       "  *p = (bf16)(((u & 0x7FFFFFFFu) > 0x7F800000u) ? ((u >> 16) | 0x40u) : r);\n}\n";
  s += "extern \"C\" __global__ __launch_bounds__(" + std::to_string(64 * groups) +
       ") void snk_fixed(const " + T + "* __restrict__ X, " + T +
       "* __restrict__ Y, int B, long long x_img, long long y_img) {\n";
  s += "  __shared__ float xs[" + std::to_string(K) + " * 64];\n";
  // the wave index, uniform over the wave: a scalar branch per group
  s += "  const int lane = threadIdx.x & 63;\n";
  s += "  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);\n";
  s += "  const long long b = (long long)blockIdx.x * 64 + lane;\n";
  s += "  const " + std::string(T) + "* Xi = X + (long long)blockIdx.y * x_img;\n";
  s += "  " + std::string(T) + "* Yi = Y + (long long)blockIdx.y * y_img;\n";
  s += "  for (int c = w; c < " + std::to_string(K) + "; c += " + std::to_string(groups) +
       ") xs[c * 64 + lane] = b < B ? ld(Xi + (long long)c * B + b) : 0.f;\n";
  s += "  __syncthreads();\n  if (b >= B) return;\n";
  s += "  float x0, x1, x2, x3;\n";
  s += "  switch (w) {\n";
  for (int g = 0; g < groups; ++g) {
    s += "  case " + std::to_string(g) + ": {\n";
    for (int32_t r0 = gs[g]; r0 < gs[g + 1]; r0 += CHUNK) {
      const int32_t r1 = std::min<int32_t>(gs[g + 1], r0 + CHUNK);
      s += "    {\n";
      for (int32_t r = r0; r < r1; ++r) s += "      float a" + std::to_string(r - r0) + " = 0.f;\n";
      // entries of the chunk, column by column
      std::map<int32_t, std::vector<std::pair<int32_t, float>>> bycol;
      for (int32_t r = r0; r < r1; ++r)
        for (int64_t k = ptr[r]; k < ptr[r + 1]; ++k)
          bycol[col[k]].push_back({r - r0, value_of(vals, dt, k)});
      // columns in order; the read of column j + PIPE is issued before the
      // entries of column j, into a rotating set of PIPE registers, so the
      // LDS latency hides behind PIPE columns of FMAs.  A compiler barrier
      // before each read keeps them in this order (else the compiler hoists
      // all of them, keeps hundreds live and spills).
      std::vector<int32_t> cols;
      for (const auto& kv : bycol) cols.push_back(kv.first);
      auto rd = [&](size_t j) {
        return "asm volatile(\"\" ::: \"memory\"); x" + std::to_string(j % PIPE) + " = xs[" +
               std::to_string(cols[j]) + " * 64 + lane];";
      };
      s += "     ";
      for (size_t j = 0; j < std::min<size_t>(PIPE, cols.size()); ++j) s += " " + rd(j);
      s += "\n";
      for (size_t j = 0; j < cols.size(); ++j) {
        const std::string xr = "x" + std::to_string(j % PIPE);
        s += "      { const float x = " + xr + ";";
        if (j + PIPE < cols.size()) s += " " + rd(j + PIPE);
        for (const auto& e : bycol[cols[j]])
          s += " a" + std::to_string(e.first) + " = __builtin_fmaf(" + f32_literal(e.second) +
               ", x, a" + std::to_string(e.first) + ");";
        s += " }\n";
      }
      for (int32_t r = r0; r < r1; ++r)
        s += "      st(Yi + " + std::to_string(r) + "LL * B + b, a" + std::to_string(r - r0) + ");\n";
      s += "    }\n";
    }
    s += "  } break;\n";
  }
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
  if (M < 1 || K < 1 || K > MAX_K || nnz < 0 || nnz > MAX_NNZ || (double)nnz > (double)M * K)
    return SNACK_E_SHAPE;
  if (nnz > 0 && (!row || !col || !vals)) return SNACK_E_NULL;
  int64_t prev = -1;
  for (int64_t k = 0; k < nnz; ++k) {
    if (row[k] < 0 || row[k] >= M || col[k] < 0 || col[k] >= K) return SNACK_E_COO_RANGE;
    const int64_t l = (int64_t)row[k] * K + col[k];
    if (l <= prev) return SNACK_E_COO_ORDER;
    prev = l;
  }
  // waves per workgroup: about 512 entries each, at most one per row
  int groups = (int)std::min<int64_t>(MAX_GROUPS, std::max<int64_t>(1, (nnz + 511) / 512));
  groups = std::min(groups, (int)M);
  snack_fixed* f = new snack_fixed();
  f->M = M;
  f->K = K;
  f->nnz = nnz;
  f->dtype = dtype;
  f->groups = groups;
  f->module = nullptr;
  f->fn = nullptr;
  f->source = generate(row, col, vals, dtype, M, K, nnz, groups);
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
  const unsigned gx = (unsigned)((B + 63) / 64);
  if (hipModuleLaunchKernel(f->fn, gx, (unsigned)images, 1, 64 * f->groups, 1, 1, 0,
                            (hipStream_t)stream, args, nullptr) != hipSuccess)
    return SNACK_E_HIP;
  return SNACK_OK;
}

snack_status snack_fixed_info(const snack_fixed* f, int32_t* groups, size_t* code_bytes,
                              size_t* source_bytes) {
  if (!f) return SNACK_E_NULL;
  if (groups) *groups = f->groups;
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
