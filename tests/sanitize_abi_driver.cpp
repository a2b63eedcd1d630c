// Host-side memory and undefined-behaviour check of the library's C ABI
// (test infrastructure). tests/test_abi_sanitized.py builds q4_api.hip with
// its host code instrumented by AddressSanitizer and UndefinedBehaviorSanitizer
// (the kernels are compiled as usual and never launched), links it with this
// driver and runs it on a machine without a GPU.
//
// The driver exercises what runs on the host before any launch: argument
// validation of every entry point (null pointers, shapes, alignment), the
// chain encoders and the product-batch encoder, whose plans are written into
// host buffers of exactly q4_chain_plan_bytes() or q4_gemm_batch_plan_bytes().
// Device pointers are stand-in addresses that the host code must never
// dereference; a dereference, a write past a plan buffer or an overflow in the
// encoders' arithmetic ends the run with the sanitizer's report. Expected
// status codes are checked as well.
#include <stdint.h>
#include <stdio.h>

#include <vector>

#include "q4.h"

namespace {

int failures = 0;
void expect(bool ok, const char* what) {
  if (!ok) {
    fprintf(stderr, "FAILED: %s\n", what);
    ++failures;
  }
}

// stand-in device addresses: distinct, 256-byte aligned, never dereferenced
uintptr_t next_addr = 0x100000000ull;
template <typename T>
T* fake(int64_t bytes) {
  const uintptr_t a = next_addr;
  next_addr += (uintptr_t)((bytes + 255) / 256 * 256 + 256);
  return reinterpret_cast<T*>(a);
}

struct Mat {
  const uint32_t* packed;
  const uint16_t* scales;
  const uint16_t* biases;
  void* y;
  int64_t n, k;
};
Mat make_mat(int64_t n, int64_t k, int rows = 1) {
  Mat m;
  m.packed = fake<uint32_t>(n * k / 2);
  m.scales = fake<uint16_t>(n * k / 16);
  m.biases = fake<uint16_t>(n * k / 16);
  m.y = fake<void>(4 * n * rows);
  m.n = n;
  m.k = k;
  return m;
}

q4_status encode(const std::vector<q4_chain_stage>& st, const std::vector<q4_chain_matrix>& mt, int rows,
                 int64_t slack = 0) {
  const int64_t bytes = q4_chain_plan_bytes((int32_t)st.size(), (int32_t)mt.size());
  if (bytes <= 0) return Q4_ERR_SHAPE;
  std::vector<unsigned char> plan((size_t)(bytes + slack));
  if (rows == 1) return q4_chain_encode(st.data(), (int32_t)st.size(), mt.data(), (int32_t)mt.size(), Q4_OUT_BF16,
                                        plan.data(), bytes + slack);
  return q4_chain_encode_rows(st.data(), (int32_t)st.size(), mt.data(), (int32_t)mt.size(), rows, Q4_OUT_F32,
                              plan.data(), bytes + slack);
}

// the temporal step: per layer q,k,v (one stage), o, gate/up, down; dependent:
// each stage's activation is the previous stage's first output
q4_status temporal_step(int layers, bool dependent, int rows) {
  std::vector<q4_chain_stage> st;
  std::vector<q4_chain_matrix> mt;
  const void* prev = nullptr;
  auto stage = [&](int64_t k, std::initializer_list<int64_t> ns) {
    q4_chain_stage s;
    s.x = dependent && prev ? static_cast<const uint16_t*>(prev) : fake<uint16_t>(2 * k * rows);
    s.k = k;
    s.first_matrix = (int32_t)mt.size();
    s.num_matrices = (int32_t)ns.size();
    for (int64_t n : ns) {
      const Mat m = make_mat(n, k, rows);
      mt.push_back({m.packed, m.scales, m.biases, m.y, m.n});
    }
    prev = mt[(size_t)s.first_matrix].y;
    st.push_back(s);
  };
  for (int l = 0; l < layers; ++l) {
    stage(4096, {4096, 4096, 4096});
    stage(4096, {4096});
    stage(4096, {11264, 11264});
    stage(11264, {4096});
  }
  return encode(st, mt, rows);
}

void check_validation() {
  const Mat m = make_mat(4096, 4096);
  const uint16_t* x = fake<uint16_t>(2 * 4096 * 64);
  const uint16_t* odd = reinterpret_cast<const uint16_t*>(reinterpret_cast<uintptr_t>(x) + 2);
  expect(q4_gemv(nullptr, m.packed, m.scales, m.biases, 4096, 4096, m.y, Q4_OUT_BF16, nullptr) == Q4_ERR_NULL,
         "gemv null x");
  expect(q4_gemv(x, m.packed, m.scales, m.biases, 4096, 4100, m.y, Q4_OUT_BF16, nullptr) == Q4_ERR_SHAPE,
         "gemv k not a multiple of 32");
  expect(q4_gemv(x, m.packed, m.scales, m.biases, 4096, 0, m.y, Q4_OUT_BF16, nullptr) == Q4_ERR_SHAPE, "gemv k 0");
  expect(q4_gemv(x, m.packed, m.scales, m.biases, -1, 4096, m.y, Q4_OUT_BF16, nullptr) == Q4_ERR_SHAPE, "gemv n < 0");
  expect(q4_gemv(odd, m.packed, m.scales, m.biases, 4096, 4096, m.y, Q4_OUT_BF16, nullptr) == Q4_ERR_ALIGN,
         "gemv misaligned x");
  expect(q4_gemv(x, m.packed, m.scales, m.biases, 0, 4096, m.y, Q4_OUT_BF16, nullptr) == Q4_OK, "gemv n == 0");
  expect(q4_gemm_small(x, 0, m.packed, m.scales, m.biases, 4096, 4096, m.y, Q4_OUT_BF16, nullptr) == Q4_ERR_SHAPE,
         "gemm m 0");
  expect(q4_gemm_small(x, Q4_MAX_M + 1, m.packed, m.scales, m.biases, 4096, 4096, m.y, Q4_OUT_BF16, nullptr) ==
             Q4_ERR_SHAPE,
         "gemm m past the limit");
  expect(q4_gemm_small(x, 16, m.packed, m.scales, m.biases, 4096, Q4_MAX_K + 32, m.y, Q4_OUT_BF16, nullptr) !=
             Q4_OK,
         "gemm k past the limit");
  expect(q4_multilinear_step(x, 1, m.packed, m.scales, m.biases, 16, 256, 4096, 16, m.y, Q4_OUT_BF16, nullptr) ==
             Q4_ERR_SHAPE,
         "multilinear step past the last");
  expect(q4_multilinear_step(x, 1, m.packed, m.scales, m.biases, (int64_t)1 << 40, 1 << 20, 4096, 0, m.y,
                             Q4_OUT_BF16, nullptr) == Q4_ERR_SHAPE,
         "multilinear rows overflow");
  expect(q4_pack(nullptr, 16, 64, fake<uint32_t>(512), fake<uint16_t>(64), fake<uint16_t>(64), nullptr) ==
             Q4_ERR_NULL,
         "pack null w");
  expect(q4_unpack(m.packed, m.scales, m.biases, 16, 48, nullptr, nullptr, nullptr) != Q4_OK, "unpack bad k");
  q4_embed_table tabs[Q4_EMBED_MAX_TABLES + 1];
  for (auto& t : tabs) {
    const Mat e = make_mat(8, 256);
    t.packed = e.packed;
    t.scales = e.scales;
    t.biases = e.biases;
    t.rows = 8;
  }
  const int32_t* tokens = fake<int32_t>(4 * 17 * 4);
  expect(q4_embed_sum(tokens, 4, tabs, Q4_EMBED_MAX_TABLES + 1, 256, fake<void>(4096), Q4_OUT_BF16, nullptr) ==
             Q4_ERR_SHAPE,
         "embed too many tables");
  expect(q4_embed_sum(tokens, 4, tabs, 17, 250, fake<void>(4096), Q4_OUT_BF16, nullptr) == Q4_ERR_SHAPE,
         "embed dim not a multiple of 32");
  expect(q4_embed_sum(nullptr, 4, tabs, 17, 256, fake<void>(4096), Q4_OUT_BF16, nullptr) == Q4_ERR_NULL,
         "embed null tokens");
  const int64_t wsb = q4_attn_workspace_bytes(32, 128);
  expect(wsb > 0, "attention workspace size");
  uint16_t* kc = fake<uint16_t>(2 * 32 * 64 * 128);
  uint16_t* vc = fake<uint16_t>(2 * 32 * 64 * 128);
  expect(q4_attn_decode(x, x, x, kc, vc, 32, 128, 64, 64, 10000.0, fake<void>(8 * 4096), Q4_OUT_F32,
                        fake<void>(wsb), wsb, nullptr) == Q4_ERR_SHAPE,
         "attention pos == cap");
  expect(q4_attn_decode(x, x, x, kc, vc, 32, 128, 64, 3, 10000.0, fake<void>(8 * 4096), Q4_OUT_F32,
                        fake<void>(wsb), wsb - 1, nullptr) != Q4_OK,
         "attention workspace too small");
  for (int s = -1; s <= 7; ++s) expect(q4_status_str(s) != nullptr, "status string");
}

void check_chains() {
  // the temporal step: 128 stages and 224 matrices, independent and dependent
  expect(temporal_step(32, false, 1) == Q4_OK, "temporal step");
  expect(temporal_step(32, true, 1) == Q4_OK, "dependent temporal step");
  expect(temporal_step(32, false, 4) == Q4_OK, "temporal step with 4 rows");
  expect(temporal_step(32, false, 5) == Q4_ERR_SHAPE, "5 rows");
  // the table limits: 96 layers are 384 stages and 672 matrices (they fit
  // with one row), 97 layers are 388 stages
  expect(temporal_step(96, false, 1) == Q4_OK, "96 layers");
  expect(temporal_step(97, false, 1) == Q4_ERR_UNSUPPORTED, "97 layers");
  {
    std::vector<q4_chain_stage> st;
    std::vector<q4_chain_matrix> mt;
    for (int s = 0; s < 385; ++s) {
      const Mat m = make_mat(1024, 1024);
      st.push_back({fake<uint16_t>(2048), 1024, s, 1});
      mt.push_back({m.packed, m.scales, m.biases, m.y, m.n});
    }
    expect(encode(st, mt, 1) == Q4_ERR_UNSUPPORTED, "385 stages");
    st.pop_back();
    mt.pop_back();
    expect(encode(st, mt, 1) == Q4_OK, "384 stages (the Depformer frame's count)");
    expect(encode(st, mt, 2) == Q4_ERR_UNSUPPORTED, "384 stages with 2 rows");
    // a plan buffer one byte short is refused, not overrun
    const int64_t bytes = q4_chain_plan_bytes((int32_t)st.size(), (int32_t)mt.size());
    std::vector<unsigned char> plan((size_t)bytes - 1);
    expect(q4_chain_encode(st.data(), (int32_t)st.size(), mt.data(), (int32_t)mt.size(), Q4_OUT_BF16, plan.data(),
                           bytes - 1) != Q4_OK,
           "plan buffer too small");
  }
  expect(q4_chain_plan_bytes(-1, 4) < 0 && q4_chain_plan_bytes(4, -1) < 0, "plan bytes of negative counts");
  // fused parts: RMSNorm, gate, residuals (in place and read by the next stage)
  {
    const int64_t k = 4096;
    std::vector<q4_chain_stage_ex> st;
    std::vector<q4_chain_matrix_ex> mt;
    void* h = fake<void>(4 * k);
    const uint16_t* g = fake<uint16_t>(2 * k);
    for (int l = 0; l < 8; ++l) {
      const Mat q = make_mat(k, k), o = make_mat(k, k), gt = make_mat(11264, k), up = make_mat(11264, k),
                d = make_mat(k, 11264);
      st.push_back({fake<uint16_t>(2 * k), k, (int32_t)mt.size(), 1, g, 1e-5, 0, 0});
      mt.push_back({q.packed, q.scales, q.biases, q.y, k, nullptr});
      st.push_back({static_cast<const uint16_t*>(q.y), k, (int32_t)mt.size(), 1, nullptr, 0.0, 0, 0});
      mt.push_back({o.packed, o.scales, o.biases, h, k, h});
      st.push_back({static_cast<const uint16_t*>(h), k, (int32_t)mt.size(), 2, g, 1e-5, 1, 0});
      mt.push_back({gt.packed, gt.scales, gt.biases, gt.y, 11264, nullptr});
      mt.push_back({up.packed, up.scales, up.biases, nullptr, 11264, nullptr});
      st.push_back({static_cast<const uint16_t*>(gt.y), 11264, (int32_t)mt.size(), 1, nullptr, 0.0, 0, 0});
      mt.push_back({d.packed, d.scales, d.biases, h, k, h});
    }
    const int64_t bytes = q4_chain_plan_bytes((int32_t)st.size(), (int32_t)mt.size());
    std::vector<unsigned char> plan((size_t)bytes);
    expect(q4_chain_encode_ex(st.data(), (int32_t)st.size(), mt.data(), (int32_t)mt.size(), 1, Q4_OUT_F32,
                              plan.data(), bytes) == Q4_OK,
           "fused decoder layers");
    // a stage whose output overlaps its own input is refused
    st[1].x = static_cast<const uint16_t*>(h);
    expect(q4_chain_encode_ex(st.data(), (int32_t)st.size(), mt.data(), (int32_t)mt.size(), 1, Q4_OUT_F32,
                              plan.data(), bytes) != Q4_OK,
           "output overlapping its own input");
  }
}

}  // namespace

// the product batch: plans written into buffers of exactly
// q4_gemm_batch_plan_bytes(), up to the item and block limits
q4_status encode_batch(const std::vector<q4_gemm_batch_item>& it, int64_t m, int64_t k, int64_t short_by = 0) {
  const int64_t blocks = q4_gemm_batch_blocks(it.data(), (int32_t)it.size());
  const int64_t bytes = q4_gemm_batch_plan_bytes((int32_t)it.size(), blocks);
  if (bytes <= 0) return Q4_ERR_SHAPE;
  std::vector<unsigned char> plan((size_t)(bytes - short_by));
  return q4_gemm_batch_encode(it.data(), (int32_t)it.size(), m, k, Q4_OUT_BF16, plan.data(), bytes - short_by);
}

q4_gemm_batch_item batch_item(int64_t n, int64_t k, int64_t m) {
  const Mat w = make_mat(n, k, (int)m);
  return {fake<uint16_t>(2 * m * k), w.packed, w.scales, w.biases, w.y, n};
}

void check_batches() {
  std::vector<q4_gemm_batch_item> step;  // the temporal step's 192 products with k = 4096
  for (int l = 0; l < 32; ++l)
    for (int64_t n : {4096, 4096, 4096, 4096, 11264, 11264}) step.push_back(batch_item(n, 4096, 16));
  expect(encode_batch(step, 16, 4096) == Q4_OK, "batch of the step's k = 4096 products");
  expect(encode_batch(step, 16, 4096, 16) == Q4_ERR_SHAPE, "batch plan buffer too small");
  expect(encode_batch(step, 4, 4096) == Q4_ERR_SHAPE, "batch of 4 rows");
  std::vector<q4_gemm_batch_item> ragged;
  for (int64_t n : {1, 15, 16, 17, 33, 1000}) ragged.push_back(batch_item(n, 96, 5));
  expect(encode_batch(ragged, 5, 96) == Q4_OK, "ragged batch");
  // 4096 items of 4096 blocks each: the 2^24-block limit exactly, then one block more
  std::vector<q4_gemm_batch_item> big;
  for (int i = 0; i < 4096; ++i) big.push_back(batch_item(65536, 256, 8));
  expect(encode_batch(big, 8, 256) == Q4_OK, "2^24 blocks");
  big.back().n += 1;
  const int64_t max_bytes = q4_gemm_batch_plan_bytes(4096, (int64_t)1 << 24);
  std::vector<unsigned char> plan((size_t)max_bytes);
  expect(q4_gemm_batch_encode(big.data(), 4096, 8, 256, Q4_OUT_BF16, plan.data(), max_bytes) == Q4_ERR_UNSUPPORTED,
         "2^24 + 1 blocks");
  big.back().n -= 1;
  big.push_back(batch_item(16, 256, 8));
  expect(q4_gemm_batch_blocks(big.data(), 4097) < 0, "4097 items");
  // run: refusals only (nothing is launched)
  std::vector<unsigned char> junk(64, 0);
  expect(q4_gemm_batch_run(junk.data(), fake<void>(64), nullptr) == Q4_ERR_SHAPE, "run of a non-plan");
  const int64_t bytes = q4_gemm_batch_plan_bytes(6, q4_gemm_batch_blocks(ragged.data(), 6));
  std::vector<unsigned char> rp((size_t)bytes);
  expect(q4_gemm_batch_encode(ragged.data(), 6, 5, 96, Q4_OUT_F32, rp.data(), bytes) == Q4_OK, "ragged plan");
  expect(q4_gemm_batch_run(rp.data(), reinterpret_cast<const char*>(fake<void>(64)) + 8, nullptr) == Q4_ERR_ALIGN,
         "run with a misaligned device plan");
}

int main() {
  check_validation();
  check_chains();
  check_batches();
  if (failures) {
    fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  printf("abi sanitized run: ok\n");
  return 0;
}
