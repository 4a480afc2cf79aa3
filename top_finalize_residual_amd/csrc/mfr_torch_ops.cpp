// Torch operators of the deferred MoE finalize: the mfr:: ops that the next
// layer's norm calls on a deferred MoE output (vLLM pull request #62174,
// Overview and Details), and the dense tail.
//
// Argument marshalling only. Each operator checks what the C ABI cannot see
// in raw pointers (dtypes, shapes, device, contiguity), takes the tensors'
// data pointers and the device's current HIP stream, and calls the C ABI of
// libmoe_finalize_rmsnorm, which validates the rest and launches the kernel.
// Written in C++ so that an eager call through torch.ops costs the
// dispatcher and the launch rather than a Python layer; the fake-tensor
// kernels that let torch.compile trace the ops are registered from Python
// (top_finalize_residual_amd/deferred.py).
//
// The fused op goes through the checked entry points with R =
// expert_out.size(0), so that a bad index from the producing layer is masked
// instead of read outside expert_out.

#include <torch/library.h>
#include <ATen/core/Tensor.h>
#include <c10/core/DeviceGuard.h>
#include <c10/hip/HIPStream.h>

#include <cstdint>

#include "moe_finalize_rmsnorm.h"

namespace {

using at::Tensor;

void check_gpu(const Tensor& t, const char* name, c10::DeviceIndex dev) {
    TORCH_CHECK_VALUE(t.is_cuda(), name, " must be on the GPU, got ", t.device());
    TORCH_CHECK_VALUE(t.get_device() == dev, "all tensors must be on one GPU, ", name, " is on ",
                      t.device());
    TORCH_CHECK_VALUE(t.is_contiguous(), name, " must be contiguous");
}

void check_dtype(const Tensor& t, const char* name, at::ScalarType want) {
    TORCH_CHECK_TYPE(t.scalar_type() == want, name, " must be ", want, ", got ", t.scalar_type());
}

void check_shape(const Tensor& t, const char* name, at::IntArrayRef want) {
    TORCH_CHECK_VALUE(t.sizes() == want, name, " has shape ", t.sizes(), ", expected ", want);
}

void check_codes(const Tensor& t, const char* name) {
    TORCH_CHECK_TYPE(t.scalar_type() == at::kFloat8_e4m3fn || t.scalar_type() == at::kByte, name,
                     " must be float8_e4m3fn or uint8, got ", t.scalar_type());
}

void check_status(int rc, const char* op) {
    TORCH_CHECK(rc == MFR_OK, op, ": ", moe_finalize_rmsnorm_strerror(rc));
}

template <typename T>
T* ptr(const Tensor& t) {
    return static_cast<T*>(t.data_ptr());
}

struct MoeShape {
    int64_t T, H, K, R;
};

// Shapes of the fused op's inputs, checked against each other, and every
// input on the GPU of expert_out.
MoeShape moe_inputs(const Tensor& expert_out, const Tensor& perm_idx, const Tensor& topk_w,
                    const Tensor& shared_out, const Tensor& residual, const Tensor& gamma) {
    check_dtype(expert_out, "expert_out", at::kBFloat16);
    check_dtype(perm_idx, "perm_idx", at::kInt);
    check_dtype(topk_w, "topk_w", at::kFloat);
    check_dtype(shared_out, "shared_out", at::kBFloat16);
    check_dtype(residual, "residual", at::kBFloat16);
    check_dtype(gamma, "gamma", at::kBFloat16);
    TORCH_CHECK_VALUE(perm_idx.dim() == 2 && gamma.dim() == 1 && expert_out.dim() == 2,
                      "perm_idx must be [T, K], gamma [H] and expert_out [R, H]");
    const MoeShape s{perm_idx.size(0), gamma.size(0), perm_idx.size(1), expert_out.size(0)};
    TORCH_CHECK_VALUE(expert_out.size(1) == s.H, "expert_out width differs from gamma length");
    check_shape(topk_w, "topk_w", {s.T, s.K});
    check_shape(shared_out, "shared_out", {s.T, s.H});
    check_shape(residual, "residual", {s.T, s.H});
    const c10::DeviceIndex dev = expert_out.is_cuda() ? expert_out.get_device() : -1;
    check_gpu(expert_out, "expert_out", dev);
    check_gpu(perm_idx, "perm_idx", dev);
    check_gpu(topk_w, "topk_w", dev);
    check_gpu(shared_out, "shared_out", dev);
    check_gpu(residual, "residual", dev);
    check_gpu(gamma, "gamma", dev);
    return s;
}

// [T, H] bf16 output on the inputs' GPU.
void bf16_output(const Tensor& t, const char* name, int64_t T, int64_t H, c10::DeviceIndex dev) {
    check_dtype(t, name, at::kBFloat16);
    check_shape(t, name, {T, H});
    check_gpu(t, name, dev);
}

// FP8 codes [T, H] and per-token scales [T] on the inputs' GPU.
void fp8_outputs(const Tensor& codes, const Tensor& scales, int64_t T, int64_t H,
                 c10::DeviceIndex dev) {
    check_codes(codes, "normed_fp8");
    check_dtype(scales, "fp8_scale", at::kFloat);
    check_shape(codes, "normed_fp8", {T, H});
    check_shape(scales, "fp8_scale", {T});
    check_gpu(codes, "normed_fp8", dev);
    check_gpu(scales, "fp8_scale", dev);
}

hipStream_t current_stream(c10::DeviceIndex dev) {
    return c10::hip::getCurrentHIPStream(dev).stream();
}

void moe_call(const Tensor& expert_out, const Tensor& perm_idx, const Tensor& topk_w,
              const Tensor& shared_out, const Tensor& residual, const Tensor& gamma, double eps,
              double scale, const Tensor& residual_out, const Tensor& normed_out) {
    const MoeShape s = moe_inputs(expert_out, perm_idx, topk_w, shared_out, residual, gamma);
    const c10::DeviceIndex dev = expert_out.get_device();
    bf16_output(residual_out, "residual_out", s.T, s.H, dev);
    bf16_output(normed_out, "normed_out", s.T, s.H, dev);
    const c10::DeviceGuard guard(expert_out.device());
    check_status(moe_finalize_rmsnorm_checked(
                     ptr<const uint16_t>(expert_out), s.R, ptr<const int32_t>(perm_idx),
                     ptr<const float>(topk_w), ptr<const uint16_t>(shared_out),
                     ptr<const uint16_t>(residual), ptr<const uint16_t>(gamma),
                     static_cast<float>(eps), static_cast<float>(scale),
                     ptr<uint16_t>(residual_out), ptr<uint16_t>(normed_out), nullptr, s.T, s.H,
                     s.K, current_stream(dev)),
                 "moe_finalize_rmsnorm");
}

void moe_fp8_call(const Tensor& expert_out, const Tensor& perm_idx, const Tensor& topk_w,
                  const Tensor& shared_out, const Tensor& residual, const Tensor& gamma,
                  double eps, double scale, const Tensor& residual_out, const Tensor& normed_fp8,
                  const Tensor& fp8_scale) {
    const MoeShape s = moe_inputs(expert_out, perm_idx, topk_w, shared_out, residual, gamma);
    const c10::DeviceIndex dev = expert_out.get_device();
    bf16_output(residual_out, "residual_out", s.T, s.H, dev);
    fp8_outputs(normed_fp8, fp8_scale, s.T, s.H, dev);
    const c10::DeviceGuard guard(expert_out.device());
    check_status(moe_finalize_rmsnorm_fp8_checked(
                     ptr<const uint16_t>(expert_out), s.R, ptr<const int32_t>(perm_idx),
                     ptr<const float>(topk_w), ptr<const uint16_t>(shared_out),
                     ptr<const uint16_t>(residual), ptr<const uint16_t>(gamma),
                     static_cast<float>(eps), static_cast<float>(scale),
                     ptr<uint16_t>(residual_out), nullptr, ptr<uint8_t>(normed_fp8),
                     ptr<float>(fp8_scale), nullptr, s.T, s.H, s.K, current_stream(dev)),
                 "moe_finalize_rmsnorm_fp8");
}

// Shapes of the dense tail's inputs, checked against each other and placed.
std::pair<int64_t, int64_t> dense_inputs(const Tensor& x, const Tensor& residual,
                                         const Tensor& gamma) {
    check_dtype(x, "x", at::kBFloat16);
    check_dtype(residual, "residual", at::kBFloat16);
    check_dtype(gamma, "gamma", at::kBFloat16);
    TORCH_CHECK_VALUE(x.dim() == 2 && gamma.dim() == 1, "x must be [T, H] and gamma [H]");
    const int64_t T = x.size(0), H = x.size(1);
    check_shape(residual, "residual", {T, H});
    check_shape(gamma, "gamma", {H});
    const c10::DeviceIndex dev = x.is_cuda() ? x.get_device() : -1;
    check_gpu(x, "x", dev);
    check_gpu(residual, "residual", dev);
    check_gpu(gamma, "gamma", dev);
    return {T, H};
}

void dense_call(const Tensor& x, const Tensor& residual, const Tensor& gamma, double eps,
                const Tensor& residual_out, const Tensor& normed_out) {
    const auto [T, H] = dense_inputs(x, residual, gamma);
    const c10::DeviceIndex dev = x.get_device();
    bf16_output(residual_out, "residual_out", T, H, dev);
    bf16_output(normed_out, "normed_out", T, H, dev);
    const c10::DeviceGuard guard(x.device());
    check_status(residual_add_rmsnorm(ptr<const uint16_t>(x), ptr<const uint16_t>(residual),
                                      ptr<const uint16_t>(gamma), static_cast<float>(eps),
                                      ptr<uint16_t>(residual_out), ptr<uint16_t>(normed_out), T,
                                      H, current_stream(dev)),
                 "residual_add_rmsnorm");
}

void dense_fp8_call(const Tensor& x, const Tensor& residual, const Tensor& gamma, double eps,
                    const Tensor& residual_out, const Tensor& normed_fp8,
                    const Tensor& fp8_scale) {
    const auto [T, H] = dense_inputs(x, residual, gamma);
    const c10::DeviceIndex dev = x.get_device();
    bf16_output(residual_out, "residual_out", T, H, dev);
    fp8_outputs(normed_fp8, fp8_scale, T, H, dev);
    const c10::DeviceGuard guard(x.device());
    check_status(residual_add_rmsnorm_fp8(ptr<const uint16_t>(x), ptr<const uint16_t>(residual),
                                          ptr<const uint16_t>(gamma), static_cast<float>(eps),
                                          ptr<uint16_t>(residual_out), nullptr,
                                          ptr<uint8_t>(normed_fp8), ptr<float>(fp8_scale), T, H,
                                          current_stream(dev)),
                 "residual_add_rmsnorm_fp8");
}

// The operators. The out-of-place forms write a separate residual_out; the
// in-place forms (trailing underscore) update the residual stream itself,
// which is then their one mutated residual argument.
void op_moe(const Tensor& expert_out, const Tensor& perm_idx, const Tensor& topk_w,
            const Tensor& shared_out, const Tensor& residual, const Tensor& gamma, double eps,
            double scale, Tensor& residual_out, Tensor& normed_out) {
    moe_call(expert_out, perm_idx, topk_w, shared_out, residual, gamma, eps, scale, residual_out,
             normed_out);
}

void op_moe_(const Tensor& expert_out, const Tensor& perm_idx, const Tensor& topk_w,
             const Tensor& shared_out, Tensor& residual, const Tensor& gamma, double eps,
             double scale, Tensor& normed_out) {
    moe_call(expert_out, perm_idx, topk_w, shared_out, residual, gamma, eps, scale, residual,
             normed_out);
}

void op_moe_fp8(const Tensor& expert_out, const Tensor& perm_idx, const Tensor& topk_w,
                const Tensor& shared_out, const Tensor& residual, const Tensor& gamma, double eps,
                double scale, Tensor& residual_out, Tensor& normed_fp8, Tensor& fp8_scale) {
    moe_fp8_call(expert_out, perm_idx, topk_w, shared_out, residual, gamma, eps, scale,
                 residual_out, normed_fp8, fp8_scale);
}

void op_moe_fp8_(const Tensor& expert_out, const Tensor& perm_idx, const Tensor& topk_w,
                 const Tensor& shared_out, Tensor& residual, const Tensor& gamma, double eps,
                 double scale, Tensor& normed_fp8, Tensor& fp8_scale) {
    moe_fp8_call(expert_out, perm_idx, topk_w, shared_out, residual, gamma, eps, scale, residual,
                 normed_fp8, fp8_scale);
}

void op_dense(const Tensor& x, const Tensor& residual, const Tensor& gamma, double eps,
              Tensor& residual_out, Tensor& normed_out) {
    dense_call(x, residual, gamma, eps, residual_out, normed_out);
}

void op_dense_(const Tensor& x, Tensor& residual, const Tensor& gamma, double eps,
               Tensor& normed_out) {
    dense_call(x, residual, gamma, eps, residual, normed_out);
}

void op_dense_fp8(const Tensor& x, const Tensor& residual, const Tensor& gamma, double eps,
                  Tensor& residual_out, Tensor& normed_fp8, Tensor& fp8_scale) {
    dense_fp8_call(x, residual, gamma, eps, residual_out, normed_fp8, fp8_scale);
}

void op_dense_fp8_(const Tensor& x, Tensor& residual, const Tensor& gamma, double eps,
                   Tensor& normed_fp8, Tensor& fp8_scale) {
    dense_fp8_call(x, residual, gamma, eps, residual, normed_fp8, fp8_scale);
}

}  // namespace

// Schemas: mutated tensors carry alias annotations, so torch sees the
// effects (functionalization, torch.compile) and graph capture records them.
TORCH_LIBRARY(mfr, m) {
    m.def("moe_finalize_rmsnorm(Tensor expert_out, Tensor perm_idx, Tensor topk_w, "
          "Tensor shared_out, Tensor residual, Tensor gamma, float eps, float scale, "
          "Tensor(a!) residual_out, Tensor(b!) normed_out) -> ()");
    m.def("moe_finalize_rmsnorm_(Tensor expert_out, Tensor perm_idx, Tensor topk_w, "
          "Tensor shared_out, Tensor(a!) residual, Tensor gamma, float eps, float scale, "
          "Tensor(b!) normed_out) -> ()");
    m.def("moe_finalize_rmsnorm_fp8(Tensor expert_out, Tensor perm_idx, Tensor topk_w, "
          "Tensor shared_out, Tensor residual, Tensor gamma, float eps, float scale, "
          "Tensor(a!) residual_out, Tensor(b!) normed_fp8, Tensor(c!) fp8_scale) -> ()");
    m.def("moe_finalize_rmsnorm_fp8_(Tensor expert_out, Tensor perm_idx, Tensor topk_w, "
          "Tensor shared_out, Tensor(a!) residual, Tensor gamma, float eps, float scale, "
          "Tensor(b!) normed_fp8, Tensor(c!) fp8_scale) -> ()");
    m.def("residual_add_rmsnorm(Tensor x, Tensor residual, Tensor gamma, float eps, "
          "Tensor(a!) residual_out, Tensor(b!) normed_out) -> ()");
    m.def("residual_add_rmsnorm_(Tensor x, Tensor(a!) residual, Tensor gamma, float eps, "
          "Tensor(b!) normed_out) -> ()");
    m.def("residual_add_rmsnorm_fp8(Tensor x, Tensor residual, Tensor gamma, float eps, "
          "Tensor(a!) residual_out, Tensor(b!) normed_fp8, Tensor(c!) fp8_scale) -> ()");
    m.def("residual_add_rmsnorm_fp8_(Tensor x, Tensor(a!) residual, Tensor gamma, float eps, "
          "Tensor(b!) normed_fp8, Tensor(c!) fp8_scale) -> ()");
}

// GPU tensors dispatch to CUDA on ROCm builds of torch. CPU tensors reach the
// same functions, which refuse them: there is no CPU implementation.
#define MFR_IMPLS(m)                                                   \
    m.impl("moe_finalize_rmsnorm", &op_moe);                           \
    m.impl("moe_finalize_rmsnorm_", &op_moe_);                         \
    m.impl("moe_finalize_rmsnorm_fp8", &op_moe_fp8);                   \
    m.impl("moe_finalize_rmsnorm_fp8_", &op_moe_fp8_);                 \
    m.impl("residual_add_rmsnorm", &op_dense);                         \
    m.impl("residual_add_rmsnorm_", &op_dense_);                       \
    m.impl("residual_add_rmsnorm_fp8", &op_dense_fp8);                 \
    m.impl("residual_add_rmsnorm_fp8_", &op_dense_fp8_)

TORCH_LIBRARY_IMPL(mfr, CUDA, m) { MFR_IMPLS(m); }
TORCH_LIBRARY_IMPL(mfr, CPU, m) { MFR_IMPLS(m); }
