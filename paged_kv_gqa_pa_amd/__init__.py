"""MI355X-native paged grouped-query decode attention."""
