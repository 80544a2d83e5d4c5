// Internal interface between the C-ABI host layer and the kernel launchers.
// Every struct here is filled only after the host layer validated the call.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

struct ScanArgs {
  const int32_t* cu;       // device [n_seqs + 1]
  int32_t n_seqs;
  int32_t n_tokens;
  const void* q;           // [T, Hqk, dk] io, token stride q_stride
  const void* k;
  const void* v;           // [T, Hv, dv] io, token stride v_stride
  const float* g;          // [T, Hv]
  const float* beta;       // [T, Hv]
  const float* init;       // [N, Hv, dv, dk] or nullptr
  const int32_t* ckpt;     // [n_ckpt] global positions, ascending
  int32_t n_ckpt;
  void* out;               // [T, Hv, dv] io, dense
  float* final_state;      // [N, Hv, dv, dk] or nullptr
  float* ckpt_buf;         // [n_ckpt, Hv, dv, dk] or nullptr
  int64_t q_stride, k_stride, v_stride;
  int32_t Hqk, Hv, dk, dv, chunk;
  int32_t bf16;            // io dtype is bf16 (else fp32)
  int32_t l2norm;
  float scale, eps;
  // the short conv fused into the scan's loads (conv_x non-null): q, k, v
  // are then unused and come from the pre-conv rows
  const void* conv_x;      // [T, conv_dim] bf16, token stride conv_x_stride
  int64_t conv_x_stride;
  const float* conv_w;     // [conv_dim, 4]
  const void* conv_state_in;   // [N, 3, conv_dim] or nullptr (zeros)
  void* conv_state_out;    // [N, 3, conv_dim], written by the scan when conv_state_own
  void* conv_ckpt;         // [n_ckpt, 3, conv_dim] or nullptr
  int32_t conv_dim;
  int32_t conv_state_own;
};

struct DecodeArgs {
  int32_t batch;
  int32_t n_tok;           // tokens per sequence (rows b * n_tok + i)
  float* snap;             // [batch, n_tok, Hv, dv, dk] or nullptr
  const void* q;
  const void* k;
  const void* v;
  const float* g;
  const float* beta;
  float* state;            // [pool, Hv, dv, dk]
  const int32_t* slot;     // [batch] or nullptr (identity)
  void* out;               // [batch, Hv, dv]
  const float* conv_w;     // [conv_dim, 4] or nullptr (q, k, v are the conv's outputs)
  void* conv_state;        // [pool, 3, conv_dim] io, with conv_w
  int32_t conv_dim;
  int64_t q_stride, k_stride, v_stride;
  int32_t Hqk, Hv, dk, dv;
  int32_t bf16;
  int32_t l2norm;
  float scale, eps;
};

struct ConvArgs {
  const int32_t* cu;
  int32_t n_seqs;
  int32_t n_tokens;
  int32_t conv_dim;
  const void* x;
  int64_t x_stride;
  const float* w;          // [conv_dim, 4]
  const void* state_in;    // [N, 3, conv_dim] or nullptr
  void* y;
  int64_t y_stride;
  void* state_out;         // [N, 3, conv_dim] or nullptr
  const int32_t* ckpt;
  int32_t n_ckpt;
  void* conv_ckpt;         // [n_ckpt, 3, conv_dim] or nullptr
  int32_t bf16;
};

struct CopyArgs {
  const void* src;
  int32_t n;
  int64_t bytes_each;
  void* dst;
  const int64_t* slot;
  int32_t host_dst;        // dst is host memory: one workgroup per item
};

hipError_t launch_prefill(const ScanArgs& a, hipStream_t stream);
hipError_t launch_prefill_recurrent(const ScanArgs& a, hipStream_t stream);
hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_conv(const ConvArgs& a, hipStream_t stream);
hipError_t launch_conv_states(const ConvArgs& a, hipStream_t stream);
hipError_t launch_snapshot_copy(const CopyArgs& a, hipStream_t stream);

}  // namespace gdn
